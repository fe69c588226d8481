// C ABI of libmsm (declared in include/msm.h): argument checks, workspace layout,
// the host side of the pipeline, and error reporting.
#include <hip/hip_runtime.h>

#include <mutex>
#include <new>
#include <vector>
#include <stdio.h>
#include <string.h>

#include "../../include/msm.h"
#include "msm_internal.hpp"

// ------------------------------------------------------------------ reduction planes
namespace msmk {

// Plane table of the bucket reduction (k_reduce.hip states the decomposition).
// log2 of the segment length: segments of 4 slots up to c = 14, 8 at c = 15 and 16, so a
// window has at most 4096 segments (group sums of at most 64 terms).
static uint32_t seg_log2(uint32_t c) { return c >= 15 ? 3u : 2u; }

plane_table make_planes(uint32_t c, uint32_t nwin) {
  plane_table pt;
  memset(&pt, 0, sizeof pt);
  const uint32_t lambda = seg_log2(c);
  const uint32_t slots = 1u << (c - 1);
  const uint32_t nseg = slots > (1u << lambda) ? slots >> lambda : 1u;
  uint32_t lgseg = 0;
  while ((1u << lgseg) < nseg) lgseg++;
  pt.nseg = nseg;
  pt.lambda = lambda;
  pt.hb = lgseg / 2;
  pt.lb = lgseg - pt.hb;
  pt.pg = nseg >= 2048 ? 6u : 5u;  // groups of at most 64 terms, at most 64 groups per plane
  pt.np = (nseg + (1u << pt.pg) - 1) >> pt.pg;
  pt.wstride = pt.np + (1u << pt.hb) + (1u << pt.lb);
  // (exponent, window, selector) of every plane
  uint32_t tmp[MAX_PLANES];
  uint32_t n = 0;
  for (uint32_t j = 0; j < nwin; j++) {
    const uint32_t phi = (j + 1 == nwin) ? c * nwin - 128 : 0;  // log2 of window_spread
    tmp[n++] = (c * j) | (j << 8);                               // the (R + T) plane
    for (uint32_t beta = 0; beta < lgseg; beta++) {
      // bit kappa of w_lo(s) - 1 = (s << lambda) >> phi is bit kappa + phi - lambda of s
      if (beta + lambda < phi) continue;
      const uint32_t kappa = beta + lambda - phi;
      tmp[n++] = (c * j + kappa) | (j << 8) | ((beta + 1) << 16);
    }
  }
  // decreasing exponent: the longest runs of doublings are dispatched first
  for (uint32_t a = 1; a < n; a++)
    for (uint32_t b = a; b > 0 && (tmp[b] & 0xffu) > (tmp[b - 1] & 0xffu); b--) {
      const uint32_t t = tmp[b];
      tmp[b] = tmp[b - 1];
      tmp[b - 1] = t;
    }
  pt.n = n;
  for (uint32_t i = 0; i < n; i++) pt.e[i] = tmp[i];
  return pt;
}

}  // namespace msmk

using namespace msmk;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, const char* detail = "") {
  snprintf(g_err, sizeof g_err, fmt, detail);
  return code;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(MSM_ERR_HIP, "HIP error: %s (" #expr ")", hipGetErrorString(e_)); \
  } while (0)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Signed c-bit digits of the GLV half-scalars (magnitudes below 2^127) need W c >= 128.
int num_windows(int c) { return (128 + c - 1) / c; }

struct Layout {
  size_t stats, halfs, pts2, counts, offsets, rank, hist_blk, poff, block_sums, sorted_idx, aff_a, aff_b,
      xz_a, xz_b, bsum, tseg, pseg, part, res, gres;
  // stream-walker buffers, sharing the pair-tree level buffers' region (one or the other
  // runs): device slot state, partial sums and their buckets, for up to Zmax slots
  size_t w_acc, w_kst, w_head, w_tail, w_head_k, w_tail_k;
  size_t Zmax;
  size_t total;
  uint32_t K, nwin, chunk, nchunk;
  size_t E_max, half;
  plane_table planes;
};

Layout plan(size_t n, int c, int S) {
  Layout L;
  L.nwin = (uint32_t)num_windows(c);
  L.K = L.nwin << (c - 1);  // 2^(c-1) bucket slots per window (signed digits)
  L.planes = make_planes((uint32_t)c, L.nwin);
  L.E_max = 2 * n * L.nwin;  // 2n GLV points
  L.half = (L.E_max + L.K) / 2 + 1;  // elements of a level >= 1 buffer
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + (bytes ? bytes : 1), 256);
    return at;
  };
  L.stats = take(sizeof(msm_stats));
  L.halfs = take(2 * n * 16);
  L.pts2 = take(2 * n * sizeof(g1a));
  L.counts = take((size_t)L.K * 4);
  L.rank = take((size_t)L.nwin * 2 * n * 4);  // rank of each (window, half-scalar) entry
  // counting-sort chunks: about 512 (chunk, window) blocks, chunks a multiple of 1024
  {
    const size_t m = 2 * n;
    size_t ch = (m * L.nwin + 511) / 512;
    ch = ch < 1024 ? 1024 : (ch + 1023) / 1024 * 1024;  // never 0 (n = 0 still plans)
    L.chunk = (uint32_t)ch;
    L.nchunk = (uint32_t)((m + ch - 1) / ch);
    if (L.nchunk == 0) L.nchunk = 1;
  }
  L.hist_blk = take((size_t)L.nwin * L.nchunk * ((size_t)1 << (c - 1)) * 4);
  // bucket offsets, then the pair offsets of every level, K + 1 words each: one scan
  // writes them all
  L.offsets = take((size_t)(MAX_LEVELS + 1) * ((size_t)L.K + 1) * 4);
  L.poff = L.offsets + ((size_t)L.K + 1) * 4;
  L.block_sums = take((size_t)(MAX_LEVELS + 1) * (scan_blocks(L.K) + 1) * 4);
  L.sorted_idx = take(L.E_max * 4);
  const size_t region = off;
  L.aff_a = take(L.half * sizeof(g1a));
  L.aff_b = take(L.half * sizeof(g1a));
  L.xz_a = take(L.half * sizeof(xyzz_st));
  L.xz_b = take(L.half * sizeof(xyzz_st));
  const size_t levels_end = off;
  off = region;
  L.Zmax = (size_t)walk_lanes(L.E_max, S) * (size_t)S;
  L.w_acc = take(L.Zmax * 64);
  L.w_kst = take(L.Zmax * 4);
  L.w_head = take(L.Zmax * sizeof(xyzz_st));
  L.w_tail = take(L.Zmax * sizeof(xyzz_st));
  L.w_head_k = take(L.Zmax * 4);
  L.w_tail_k = take(L.Zmax * 4);
  if (off < levels_end) off = levels_end;
  L.bsum = take((size_t)L.K * sizeof(xyzz_st));
  L.tseg = take((size_t)L.nwin * L.planes.nseg * sizeof(xyzz_st));
  L.pseg = take((size_t)L.nwin * L.planes.nseg * sizeof(xyzz_st));
  L.part = take((size_t)L.nwin * L.planes.wstride * sizeof(xyzz_st));
  L.res = take((size_t)L.planes.n * sizeof(xyzz_st));
  L.gres = take((size_t)MAX_PLANE_GROUPS * sizeof(xyzz_st));
  L.total = off;
  return L;
}

// plan() of the last shape asked for on this thread (planning takes microseconds, which a
// run would otherwise spend before its first launch, twice).
Layout plan_cached(size_t n, int c, int S) {
  thread_local Layout L;
  thread_local size_t kn = SIZE_MAX;
  thread_local int kc = 0, kS = 0;
  if (n != kn || c != kc || S != kS) {
    L = plan(n, c, S);
    kn = n;
    kc = c;
    kS = S;
  }
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_run_args(const msm_g1_affine* pts, const uint32_t* sc, size_t n, int c, int S,
                   int sched, int verify, const msm_g1_affine* out) {
  if (c < 1 || c > 16) return fail(MSM_ERR_ARG, "window c must be in 1..16%s");
  if (S != 4 && S != 8 && S != 16 && S != 32) return fail(MSM_ERR_ARG, "S must be 4, 8, 16 or 32%s");
  if (sched != MSM_SCHED_PAIR_TREE && sched != MSM_SCHED_WALKER)
    return fail(MSM_ERR_ARG, "sched must be MSM_SCHED_PAIR_TREE (0) or MSM_SCHED_WALKER (1)%s");
  if (verify != 0 && verify != 1) return fail(MSM_ERR_ARG, "verify must be 0 or 1%s");
  if (n > MSM_MAX_N) return fail(MSM_ERR_ARG, "n exceeds MSM_MAX_N%s");
  if ((uint64_t)2 * n * (uint64_t)num_windows(c) >= ((uint64_t)1 << 32))
    return fail(MSM_ERR_ARG, "2 n ceil(128 / c) bucket entries exceed 32-bit offsets; raise c%s");
  if (!out) return fail(MSM_ERR_ARG, "d_out is NULL%s");
  if (n && (!pts || !sc)) return fail(MSM_ERR_ARG, "points or scalars pointer is NULL%s");
  if (!aligned(pts, 16) || !aligned(sc, 16) || !aligned(out, 16))
    return fail(MSM_ERR_ARG, "points, scalars and d_out must be 16-byte aligned%s");
  return MSM_OK;
}

// Workspace of msm_run_noalloc: a fixed device array, one copy per GPU the library
// runs on, held until the process ends. Host code never uses its name as an address:
// each device's copy is looked up once with hipGetSymbolAddress (noalloc_scratch_of).
constexpr size_t NOALLOC_MAX_BYTES = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_MAX_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};
hipError_t g_scratch_err[NOALLOC_MAX_DEVICES] = {};
bool g_scratch_done[NOALLOC_MAX_DEVICES] = {};

// Device address of this device's copy of scratch, looked up on the first call per
// device (with that device current); nullptr and *err set when the lookup failed.
void* noalloc_scratch_of(int device, hipError_t* err) {
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (device < 0 || device >= NOALLOC_MAX_DEVICES) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  if (!g_scratch_done[device]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_err[device] = e;
    g_scratch_ptr[device] = (e == hipSuccess) ? ptr : nullptr;
    g_scratch_done[device] = true;
  }
  *err = g_scratch_err[device];
  return g_scratch_ptr[device];
}

}  // namespace

enum Phase { PH_SORT = 0, PH_ACCUM = 1, PH_LEVEL = 2, PH_REDUCE = 3, PH_FINAL = 4, PH_XYZZ = 5 };

struct Span {
  int phase;
  size_t e0, e1;
};

struct msm_ctx {
  int device = 0;
  int affine_levels = 1;  // leading pair-tree levels done with batched affine adds
  int walker_device_state = 1;  // stream walker: accumulators on the device (1) or private (0)
  int prefix_store = 0;  // batched-affine level: prefix products private (0) / LDS (1), +2 dx cache
  int scalar_form = 0;   // scalars as integers (0) or Montgomery-form F_r elements (1)
  void* ws = nullptr;
  size_t ws_bytes = 0;
  msm_stats* host_stats = nullptr;  // pinned: the plan, then the result's verify flag
  msm_g1_affine* d_result = nullptr;  // device result buffer of the synchronous msm()
  hipEvent_t plan_ready = nullptr;   // the plan's copy to host_stats has completed
  hipEvent_t done = nullptr;         // the last kernel of the previous call has run
  bool has_done = false;
  hipStream_t done_stream = nullptr;  // the stream done was last recorded on
  void* noalloc_ws = nullptr;        // this device's fixed workspace of msm_run_noalloc
  // phase timing: 0 off, 1 the batched-affine level kernels only, 2 every phase
  int timing = 0;
  std::vector<hipEvent_t> events;
  size_t ev_used = 0;
  std::vector<Span> spans;
  int runs = 0, level_launches = 0;
  uint64_t level_pairs = 0, level_lanes = 0;
};

namespace {

// Record an event on the stream; returns its index, or SIZE_MAX on failure.
size_t mark(msm_ctx* ctx, hipStream_t st) {
  if (ctx->ev_used == ctx->events.size()) {
    hipEvent_t e;
    // timing only: no system-scope cache writeback when it is recorded, which would
    // otherwise stall the kernel after it
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return SIZE_MAX;
    ctx->events.push_back(e);
  }
  size_t i = ctx->ev_used++;
  if (hipEventRecord(ctx->events[i], st) != hipSuccess) return SIZE_MAX;
  return i;
}

struct PhaseMark {
  msm_ctx* ctx;
  hipStream_t st;
  int phase;
  int level;  // the context's timing level, or 0 where no event may be created
  size_t e0 = SIZE_MAX;
  // level 1 brackets the batched-affine accumulate kernels and the combine, level 2
  // every phase
  bool on() const { return level >= 2 || (level == 1 && (phase == PH_LEVEL || phase == PH_FINAL)); }
  PhaseMark(msm_ctx* c, hipStream_t s, int ph, int lvl) : ctx(c), st(s), phase(ph), level(lvl) {
    if (on()) e0 = mark(ctx, st);
  }
  void end() {
    if (on() && e0 != SIZE_MAX) {
      size_t e1 = mark(ctx, st);
      if (e1 != SIZE_MAX) ctx->spans.push_back({phase, e0, e1});
    }
    e0 = SIZE_MAX;
  }
};

}  // namespace

namespace {

// The whole MSM on stream st with workspace ws (laid out by L); arguments checked.
int run_pipeline(msm_ctx* ctx, const g1a* d_points, const uint32_t* d_scalars, size_t n, int c,
                 int S, int sched, int verify, char* ws, const Layout& L, hipStream_t st,
                 g1a* d_out, bool timed) {
  const int tl = timed ? ctx->timing : 0;
  // calls on one context are ordered even across streams: wait for the previous one (on
  // the same stream, stream order already does)
  if (ctx->has_done && ctx->done_stream != st) HIP_TRY(hipStreamWaitEvent(st, ctx->done, 0));
  // marks the last kernel queued so far: at the end, and before an error return once
  // kernels are queued
  auto record_done = [&]() -> hipError_t {
    hipError_t e = hipEventRecord(ctx->done, st);
    if (e == hipSuccess) {
      ctx->has_done = true;
      ctx->done_stream = st;
    }
    return e;
  };
  if (n == 0) {
    HIP_TRY(launch_fill((uint32_t*)d_out, sizeof(msm_g1_affine) / 4, 0, st));
    HIP_TRY(record_done());
    return MSM_OK;
  }
  msm_stats* stats = (msm_stats*)(ws + L.stats);
  uint32_t* halfs = (uint32_t*)(ws + L.halfs);
  g1a* pts2 = (g1a*)(ws + L.pts2);
  uint32_t* counts = (uint32_t*)(ws + L.counts);
  uint32_t* offsets = (uint32_t*)(ws + L.offsets);
  uint32_t* rank = (uint32_t*)(ws + L.rank);
  uint32_t* hist_blk = (uint32_t*)(ws + L.hist_blk);
  uint32_t* poff = (uint32_t*)(ws + L.poff);
  uint32_t* block_sums = (uint32_t*)(ws + L.block_sums);
  uint32_t* sorted_idx = (uint32_t*)(ws + L.sorted_idx);
  g1a* aff[2] = {(g1a*)(ws + L.aff_a), (g1a*)(ws + L.aff_b)};
  xyzz_st* xz[2] = {(xyzz_st*)(ws + L.xz_a), (xyzz_st*)(ws + L.xz_b)};
  xyzz_st* bsum = (xyzz_st*)(ws + L.bsum);
  xyzz_st* tseg = (xyzz_st*)(ws + L.tseg);
  xyzz_st* pseg = (xyzz_st*)(ws + L.pseg);
  xyzz_st* part = (xyzz_st*)(ws + L.part);
  xyzz_st* res = (xyzz_st*)(ws + L.res);
  xyzz_st* gres = (xyzz_st*)(ws + L.gres);
  const g1a* pts = pts2;  // 2n points: P_i and phi(P_i)
  uint32_t n32 = (uint32_t)n, m32 = 2 * (uint32_t)n, c32 = (uint32_t)c;

  // Levels the plan can require: a bucket holds at most one entry per half-scalar.
  int level_bound = 0;
  while (level_bound < MAX_LEVELS && ((uint64_t)1 << level_bound) < (uint64_t)m32) level_bound++;

  // decompose + count, offsets, plan; the plan is copied to the host as soon as the
  // counts are known, and the scatter, bucket init and the pair offsets of every level
  // the plan can require are queued behind it, so the GPU keeps working while the host
  // waits for the plan
  PhaseMark ph_sort(ctx, st, PH_SORT, tl);
  HIP_TRY(launch_fill((uint32_t*)stats, sizeof(msm_stats) / 4, 0, st));
  HIP_TRY(launch_glv_prep(d_points, d_scalars, n32, pts2, halfs, stats, verify, ctx->scalar_form, st));
  HIP_TRY(launch_hist(halfs, m32, c32, L.nwin, L.chunk, L.nchunk, hist_blk, counts, rank, stats, st));
  // bucket offsets (scan level -1) and, for the pair tree, the pair offsets of every level
  // it can need (level l at poff + l (K + 1)) in one set of scan launches
  HIP_TRY(launch_scan(counts, L.K, -1, 1 + (sched == MSM_SCHED_PAIR_TREE ? level_bound : 0),
                      block_sums, offsets, (size_t)L.K + 1, &stats->max_count, st));
  HIP_TRY(hipMemcpyAsync(ctx->host_stats, stats, sizeof(msm_stats), hipMemcpyDeviceToHost, st));
  HIP_TRY(hipEventRecord(ctx->plan_ready, st));
  HIP_TRY(launch_scatter(halfs, m32, c32, L.nwin, L.chunk, L.nchunk, offsets, hist_blk, rank,
                         sorted_idx, st));
  ph_sort.end();
  PhaseMark ph_acc(ctx, st, PH_ACCUM, tl);
  HIP_TRY(launch_bucket_init(counts, offsets, L.K, sorted_idx, pts, bsum, st));
  uint32_t* const poff_all = poff;
  {
    const hipError_t e = hipEventSynchronize(ctx->plan_ready);
    if (e != hipSuccess) {
      (void)record_done();
      return fail(MSM_ERR_HIP, "HIP error: %s (waiting for the plan)", hipGetErrorString(e));
    }
  }
  const msm_stats hs = *ctx->host_stats;
  if (hs.range_flag || hs.bad_point) HIP_TRY(record_done());
  if (hs.range_flag) return fail(MSM_ERR_RANGE, "GLV half-scalar out of bound (internal error)%s");
  if (hs.bad_point)
    return fail(MSM_ERR_OFF_CURVE, "an input point is not on the curve or not reduced below p%s");

  if (sched == MSM_SCHED_WALKER) {
    // accumulate: the stream walker over the E sorted entries
    walk_args wa;
    wa.pts = pts;
    wa.idx = sorted_idx;
    wa.offsets = offsets;
    wa.K = L.K;
    wa.E = hs.total;
    wa.T = walk_lanes(hs.total, S);
    wa.L = (uint32_t)(((uint64_t)hs.total + (uint64_t)wa.T * S - 1) / ((uint64_t)wa.T * S));
    wa.acc = (uint32_t*)(ws + L.w_acc);
    wa.kst = (uint32_t*)(ws + L.w_kst);
    wa.bsum = bsum;
    wa.head = (xyzz_st*)(ws + L.w_head);
    wa.tail = (xyzz_st*)(ws + L.w_tail);
    wa.head_k = (uint32_t*)(ws + L.w_head_k);
    wa.tail_k = (uint32_t*)(ws + L.w_tail_k);
    // pair passes for the most split bucket: it covers at most ceil(max / L) + 1 chunks
    const uint64_t span = ((uint64_t)hs.max_count + wa.L - 1) / (wa.L ? wa.L : 1) + 1;
    uint32_t passes = 0;
    while (((uint64_t)1 << passes) < span) passes++;
    if (hs.total) {
      PhaseMark ph_lvl(ctx, st, PH_LEVEL, tl);
      HIP_TRY(launch_walk(S, ctx->walker_device_state != 0, wa, st));
      ph_lvl.end();
      HIP_TRY(launch_walk_merge(S, wa, passes, st));
      if (tl) {
        ctx->level_launches++;
        ctx->level_pairs += hs.total;  // entries walked (one add each, or a bucket start)
        ctx->level_lanes += (uint64_t)wa.T * wa.L;  // one inversion per lane and step
      }
    }
  }
  // accumulate: pair-tree levels until every bucket holds one point
  int levels = 0;
  while (sched == MSM_SCHED_PAIR_TREE && levels < level_bound && ((uint64_t)1 << levels) < hs.max_count)
    levels++;
  for (int l = 0; l < levels; l++) {
    uint32_t np = hs.pairs[l];
    if (np == 0) continue;
    const uint32_t* lvl_poff = poff_all + (size_t)l * (L.K + 1);
    const uint32_t* idx = (l == 0) ? sorted_idx : nullptr;
    const int La = ctx->affine_levels < 0 ? MAX_LEVELS : ctx->affine_levels;
    if (l < La) {
      // batched affine adds, S per lane sharing one inversion
      const g1a* in = (l == 0) ? pts : aff[(l - 1) & 1];
      PhaseMark ph_lvl(ctx, st, PH_LEVEL, tl);
      HIP_TRY(launch_level(S, ctx->prefix_store, in, idx, aff[l & 1], bsum, counts, offsets,
                           lvl_poff, L.K, np, l, st));
      ph_lvl.end();
      if (tl) {
        ctx->level_launches++;
        ctx->level_pairs += np;
        ctx->level_lanes += (np + S - 1) / S;
      }
    } else {
      // XYZZ adds, one pair per lane; the first such level reads affine input
      const bool in_aff = (l == La) || l == 0;
      const void* in = (l == 0) ? (const void*)pts
                       : in_aff ? (const void*)aff[(l - 1) & 1] : (const void*)xz[(l - 1) & 1];
      PhaseMark ph_lvl(ctx, st, PH_XYZZ, tl);
      HIP_TRY(launch_level_xyzz(in_aff, in, idx, xz[l & 1], bsum, counts, offsets, lvl_poff, L.K,
                                np, l, st));
      ph_lvl.end();
    }
  }
  ph_acc.end();

  // segment and plane sums, doubling runs, plane sum
  PhaseMark ph_red(ctx, st, PH_REDUCE, tl);
  HIP_TRY(launch_reduce(bsum, c32, L.nwin, L.planes, tseg, pseg, part, st));
  ph_red.end();
  PhaseMark ph_fin(ctx, st, PH_FINAL, tl);
  HIP_TRY(launch_final(part, L.planes, res, gres, stats->join, d_out, st));
  ph_fin.end();
  if (verify) HIP_TRY(launch_verify_point(d_out, &stats->bad_out, st));
  HIP_TRY(record_done());
  if (tl) ctx->runs++;
  if (verify) {
    HIP_TRY(hipMemcpyAsync(&ctx->host_stats->bad_out, &stats->bad_out, 4, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    if (ctx->host_stats->bad_out) return fail(MSM_ERR_OFF_CURVE, "the result is not on the curve%s");
  }
  return MSM_OK;
}

}  // namespace

extern "C" {

int msm_version(void) { return 300; }

const char* msm_last_error(void) { return g_err; }

size_t msm_workspace_bytes(size_t n, int c, int S) {
  if (c < 1 || c > 16 || n > MSM_MAX_N) return 0;
  if ((uint64_t)2 * n * (uint64_t)num_windows(c) >= ((uint64_t)1 << 32)) return 0;
  if (S != 4 && S != 8 && S != 16 && S != 32) return 0;
  return plan_cached(n, c, S).total;
}

int msm_ctx_create(int device, msm_ctx** out) {
  if (!out) return fail(MSM_ERR_ARG, "out is NULL%s");
  *out = nullptr;
  int ndev = 0;
  HIP_TRY(hipGetDeviceCount(&ndev));
  if (device < 0 || device >= ndev) return fail(MSM_ERR_ARG, "no such device%s");
  msm_ctx* ctx = new (std::nothrow) msm_ctx;
  if (!ctx) return fail(MSM_ERR_OOM, "host allocation failed%s");
  ctx->device = device;
  int rc = MSM_OK;
  if (hipSetDevice(device) != hipSuccess) {
    rc = fail(MSM_ERR_HIP, "hipSetDevice failed%s");
  } else if (hipHostMalloc((void**)&ctx->host_stats, sizeof(msm_stats), hipHostMallocDefault) !=
             hipSuccess) {
    ctx->host_stats = nullptr;
    rc = fail(MSM_ERR_OOM, "pinned host allocation failed%s");
  } else if (hipMalloc((void**)&ctx->d_result, 256) != hipSuccess) {
    ctx->d_result = nullptr;
    rc = fail(MSM_ERR_OOM, "device allocation failed%s");
  } else if (hipEventCreateWithFlags(&ctx->plan_ready, hipEventDisableTiming) != hipSuccess ||
             // device-scope release: it orders later calls' kernels and tells the host
             // the workspace is free, and nothing on the host reads what came before it
             hipEventCreateWithFlags(&ctx->done, hipEventDisableTiming | hipEventReleaseToDevice) !=
                 hipSuccess) {
    rc = fail(MSM_ERR_HIP, "event creation failed%s");
  } else {
    // set-up of msm_run_noalloc: this device's copy of its fixed workspace; a failed
    // lookup only disables that entry point (it reports the error)
    hipError_t e;
    ctx->noalloc_ws = noalloc_scratch_of(device, &e);
  }
  if (rc != MSM_OK) {
    msm_ctx_destroy(ctx);
    return rc;
  }
  *out = ctx;
  return MSM_OK;
}

void msm_ctx_destroy(msm_ctx* ctx) {
  if (!ctx) return;
  (void)hipSetDevice(ctx->device);
  if (ctx->has_done) (void)hipEventSynchronize(ctx->done);
  for (hipEvent_t e : ctx->events) (void)hipEventDestroy(e);
  if (ctx->plan_ready) (void)hipEventDestroy(ctx->plan_ready);
  if (ctx->done) (void)hipEventDestroy(ctx->done);
  if (ctx->ws) (void)hipFree(ctx->ws);
  if (ctx->d_result) (void)hipFree(ctx->d_result);
  if (ctx->host_stats) (void)hipHostFree(ctx->host_stats);
  delete ctx;
}

int msm_run(msm_ctx* ctx, const msm_g1_affine* d_points, const uint32_t* d_scalars, size_t n,
            int c, int S, int sched, int verify, void* d_workspace, size_t workspace_bytes,
            void* stream, msm_g1_affine* d_out) {
  if (!ctx) return fail(MSM_ERR_ARG, "ctx is NULL%s");
  int rc = check_run_args(d_points, d_scalars, n, c, S, sched, verify, d_out);
  if (rc) return rc;
  const Layout L = plan_cached(n, c, S);
  if (d_workspace && (workspace_bytes < L.total || !aligned(d_workspace, 256)))
    return fail(MSM_ERR_ARG, "workspace smaller than msm_workspace_bytes() or not 256-byte aligned%s");
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(ctx->device));
  char* ws = (char*)d_workspace;
  if (!ws && n) {
    if (ctx->ws_bytes < L.total) {
      if (ctx->ws) {
        // the previous call may still be using the old workspace on another stream
        if (ctx->has_done) HIP_TRY(hipEventSynchronize(ctx->done));
        HIP_TRY(hipFree(ctx->ws));
        ctx->ws = nullptr;
        ctx->ws_bytes = 0;
      }
      if (hipMalloc(&ctx->ws, L.total) != hipSuccess) {
        ctx->ws = nullptr;
        return fail(MSM_ERR_OOM, "workspace allocation failed%s");
      }
      ctx->ws_bytes = L.total;
    }
    ws = (char*)ctx->ws;
  }
  return run_pipeline(ctx, (const g1a*)d_points, d_scalars, n, c, S, sched, verify, ws, L, st,
                      (g1a*)d_out, true);
}

int msm_run_noalloc(msm_ctx* ctx, const msm_g1_affine* d_points, const uint32_t* d_scalars,
                    size_t n, int c, int S, int sched, int verify, void* stream,
                    msm_g1_affine* d_out) {
  if (!ctx) return fail(MSM_ERR_ARG, "ctx is NULL%s");
  int rc = check_run_args(d_points, d_scalars, n, c, S, sched, verify, d_out);
  if (rc) return rc;
  const Layout L = plan_cached(n, c, S);
  if (L.total > NOALLOC_MAX_BYTES)
    return fail(MSM_ERR_ARG,
                "msm_workspace_bytes(n, c, S) exceeds the fixed workspace of msm_run_noalloc "
                "(MSM_NOALLOC_MAX_BYTES); use msm_run%s");
  if (!ctx->noalloc_ws) {
    hipError_t e;
    (void)noalloc_scratch_of(ctx->device, &e);
    return fail(MSM_ERR_HIP, "HIP error: %s (looking up the fixed workspace)", hipGetErrorString(e));
  }
  HIP_TRY(hipSetDevice(ctx->device));
  return run_pipeline(ctx, (const g1a*)d_points, d_scalars, n, c, S, sched, verify,
                      (char*)ctx->noalloc_ws, L, (hipStream_t)stream, (g1a*)d_out, false);
}

int msm_ctx_set_affine_levels(msm_ctx* ctx, int levels) {
  if (!ctx) return fail(MSM_ERR_ARG, "ctx is NULL%s");
  if (levels < -1 || levels > MAX_LEVELS) return fail(MSM_ERR_ARG, "levels must be -1 .. 32%s");
  ctx->affine_levels = levels;
  return MSM_OK;
}

int msm_ctx_set_walker_state(msm_ctx* ctx, int device_state) {
  if (!ctx) return fail(MSM_ERR_ARG, "ctx is NULL%s");
  if (device_state != 0 && device_state != 1) return fail(MSM_ERR_ARG, "device_state must be 0 or 1%s");
  ctx->walker_device_state = device_state;
  return MSM_OK;
}

int msm_ctx_set_prefix_store(msm_ctx* ctx, int store) {
  if (!ctx) return fail(MSM_ERR_ARG, "ctx is NULL%s");
  if (store < 0 || store > 4) return fail(MSM_ERR_ARG, "store must be in 0..4%s");
  ctx->prefix_store = store;
  return MSM_OK;
}

int msm_ctx_set_scalar_form(msm_ctx* ctx, int form) {
  if (!ctx) return fail(MSM_ERR_ARG, "ctx is NULL%s");
  if (form != MSM_SCALARS_INTEGER && form != MSM_SCALARS_MONTGOMERY)
    return fail(MSM_ERR_ARG, "form must be MSM_SCALARS_INTEGER or MSM_SCALARS_MONTGOMERY%s");
  ctx->scalar_form = form;
  return MSM_OK;
}

int msm_ctx_set_timing(msm_ctx* ctx, int enable) {
  if (!ctx) return fail(MSM_ERR_ARG, "ctx is NULL%s");
  if (enable < 0 || enable > 2) return fail(MSM_ERR_ARG, "timing level must be 0, 1 or 2%s");
  ctx->timing = enable;
  return MSM_OK;
}

int msm_ctx_timing_read(msm_ctx* ctx, msm_timing* out) {
  if (!ctx || !out) return fail(MSM_ERR_ARG, "NULL argument%s");
  memset(out, 0, sizeof *out);
  HIP_TRY(hipSetDevice(ctx->device));
  double* slot[6] = {&out->sort_ms, &out->accumulate_ms, &out->level_kernel_ms, &out->reduce_ms,
                     &out->final_ms, &out->xyzz_level_ms};
  for (const Span& sp : ctx->spans) {
    HIP_TRY(hipEventSynchronize(ctx->events[sp.e1]));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, ctx->events[sp.e0], ctx->events[sp.e1]));
    *slot[sp.phase] += ms;
  }
  out->runs = ctx->runs;
  out->level_launches = ctx->level_launches;
  out->level_pairs = ctx->level_pairs;
  out->level_lanes = ctx->level_lanes;
  ctx->spans.clear();
  ctx->ev_used = 0;
  ctx->runs = ctx->level_launches = 0;
  ctx->level_pairs = ctx->level_lanes = 0;
  return MSM_OK;
}

int msm(const msm_g1_affine* d_points, const uint32_t* d_scalars, size_t n, int c,
        msm_g1_affine* h_out) {
  if (!h_out) return fail(MSM_ERR_ARG, "h_out is NULL%s");
  int rc = check_run_args(d_points, d_scalars, n, c, 8, MSM_SCHED_PAIR_TREE, 0,
                          (const msm_g1_affine*)16);
  if (rc) return rc;
  static std::mutex mu;
  static msm_ctx* ctxs[64] = {};
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(MSM_ERR_ARG, "device index out of range%s");
  std::lock_guard<std::mutex> g(mu);
  if (!ctxs[dev]) {
    rc = msm_ctx_create(dev, &ctxs[dev]);
    if (rc) return rc;
  }
  msm_ctx* ctx = ctxs[dev];
  rc = msm_run(ctx, d_points, d_scalars, n, c, 8, MSM_SCHED_PAIR_TREE, 0, nullptr, 0, nullptr,
               ctx->d_result);
  if (rc == MSM_OK) {
    hipError_t e = hipMemcpy(h_out, ctx->d_result, sizeof(msm_g1_affine), hipMemcpyDeviceToHost);
    if (e != hipSuccess) rc = fail(MSM_ERR_HIP, "HIP error: %s (copy result)", hipGetErrorString(e));
  }
  return rc;
}

int msm_g1_from_scalars(const uint32_t* d_k, size_t n, msm_g1_affine* d_out, void* stream) {
  if (n > MSM_MAX_N) return fail(MSM_ERR_ARG, "n exceeds MSM_MAX_N%s");
  if (n && (!d_k || !d_out)) return fail(MSM_ERR_ARG, "NULL pointer%s");
  if (!aligned(d_k, 16) || !aligned(d_out, 16)) return fail(MSM_ERR_ARG, "pointers must be 16-byte aligned%s");
  HIP_TRY(launch_from_scalars(d_k, (uint32_t)n, (g1a*)d_out, (hipStream_t)stream));
  return MSM_OK;
}

int msm_test_fp(int op, const uint32_t* d_a, const uint32_t* d_b, uint32_t* d_out, size_t n,
                void* stream) {
  if (op < 0 || op > 8) return fail(MSM_ERR_ARG, "op must be in 0..8%s");
  if (n > MSM_MAX_N) return fail(MSM_ERR_ARG, "n exceeds MSM_MAX_N%s");
  bool binary = (op <= 2);
  if (n && (!d_a || !d_out || (binary && !d_b))) return fail(MSM_ERR_ARG, "NULL pointer%s");
  if (!aligned(d_a, 4) || !aligned(d_b, 4) || !aligned(d_out, 4))
    return fail(MSM_ERR_ARG, "pointers must be 4-byte aligned%s");
  HIP_TRY(launch_test_fp(op, d_a, binary ? d_b : nullptr, d_out, (uint32_t)n, (hipStream_t)stream));
  return MSM_OK;
}

int msm_test_fp_mul(const uint32_t* d_a, const uint32_t* d_b, uint32_t* d_out, size_t n, void* stream) {
  return msm_test_fp(0, d_a, d_b, d_out, n, stream);
}

int msm_test_fp_add(const uint32_t* d_a, const uint32_t* d_b, uint32_t* d_out, size_t n, void* stream) {
  return msm_test_fp(1, d_a, d_b, d_out, n, stream);
}

int msm_test_fp_sub(const uint32_t* d_a, const uint32_t* d_b, uint32_t* d_out, size_t n, void* stream) {
  return msm_test_fp(2, d_a, d_b, d_out, n, stream);
}

int msm_test_fp_sqr(const uint32_t* d_a, uint32_t* d_out, size_t n, void* stream) {
  return msm_test_fp(3, d_a, nullptr, d_out, n, stream);
}

int msm_test_fp_inv(const uint32_t* d_a, uint32_t* d_out, size_t n, void* stream) {
  return msm_test_fp(4, d_a, nullptr, d_out, n, stream);
}

int msm_test_row(int op, const uint32_t* d_a, const uint32_t* d_b, uint32_t* d_out, size_t n,
                 uint32_t d, void* stream) {
  if (op < 0 || op > 9) return fail(MSM_ERR_ARG, "op must be in 0..9%s");
  if (n > MSM_MAX_N) return fail(MSM_ERR_ARG, "n exceeds MSM_MAX_N%s");
  if ((op == 5 || op == 6) && n != 4) return fail(MSM_ERR_ARG, "the latency probe takes n = 4%s");
  if ((op == 3 || op == 4) && d > 4096) return fail(MSM_ERR_ARG, "d must be at most 4096%s");
  const bool binary = op <= 2 || op == 5 || op == 6 || op == 7;
  if (n && (!d_a || !d_out || (binary && !d_b))) return fail(MSM_ERR_ARG, "NULL pointer%s");
  if (!aligned(d_a, 4) || !aligned(d_b, 4) || !aligned(d_out, 4))
    return fail(MSM_ERR_ARG, "pointers must be 4-byte aligned%s");
  HIP_TRY(launch_test_row(op, d_a, binary ? d_b : nullptr, d_out, (uint32_t)n, d, (hipStream_t)stream));
  return MSM_OK;
}

int msm_test_issue_rate(int op, uint32_t blocks, uint32_t iters, uint32_t* d_out, void* stream) {
  if (op < 0 || op > 2) return fail(MSM_ERR_ARG, "op must be 0, 1 or 2%s");
  if (blocks == 0 || blocks > (1u << 20) || iters == 0) return fail(MSM_ERR_ARG, "blocks or iters out of range%s");
  if (!d_out || !aligned(d_out, 4)) return fail(MSM_ERR_ARG, "d_out is NULL or misaligned%s");
  HIP_TRY(launch_test_rate(op, blocks, iters, 0x9e3779b9u, d_out, (hipStream_t)stream));
  return MSM_OK;
}

int msm_test_glv(const uint32_t* d_scalars, size_t n, uint32_t* d_halfs, void* stream) {
  if (n > MSM_MAX_N) return fail(MSM_ERR_ARG, "n exceeds MSM_MAX_N%s");
  if (n && (!d_scalars || !d_halfs)) return fail(MSM_ERR_ARG, "NULL pointer%s");
  if (!aligned(d_scalars, 16) || !aligned(d_halfs, 16))
    return fail(MSM_ERR_ARG, "pointers must be 16-byte aligned%s");
  if (n) HIP_TRY(launch_test_glv(d_scalars, (uint32_t)n, d_halfs, (hipStream_t)stream));
  return MSM_OK;
}

int msm_test_batched_add(const msm_g1_affine* d_a, const msm_g1_affine* d_b,
                         msm_g1_affine* d_out, size_t n, int S, void* stream) {
  if (S != 4 && S != 8 && S != 16 && S != 32) return fail(MSM_ERR_ARG, "S must be 4, 8, 16 or 32%s");
  if (n > MSM_MAX_N) return fail(MSM_ERR_ARG, "n exceeds MSM_MAX_N%s");
  if (n && (!d_a || !d_b || !d_out)) return fail(MSM_ERR_ARG, "NULL pointer%s");
  if (!aligned(d_a, 16) || !aligned(d_b, 16) || !aligned(d_out, 16))
    return fail(MSM_ERR_ARG, "pointers must be 16-byte aligned%s");
  HIP_TRY(launch_test_pair_add(S, (const g1a*)d_a, (const g1a*)d_b, (g1a*)d_out, (uint32_t)n,
                               (hipStream_t)stream));
  return MSM_OK;
}

}  // extern "C"
