/*
 * msm.h - C ABI of libmsm, an MI355X (gfx950) multi-scalar multiplication over
 * BN254 G1:
 *
 *     Q = sum_{i < n} s_i * P_i
 *
 * The method is the bucket (Pippenger) MSM of aztec-packages PR #23738 / #23736 /
 * #23520 ("bb/msm"): scalars are cut into c-bit windows (c = 13 at n = 2^16 in
 * PR #23520, "Measurements"), (bucket, point) pairs are sorted into per-bucket lists
 * (the sorted_bucket_list / sorted_count_list of PR #23738, "What would actually
 * win"), each bucket is summed with affine additions in batches of S that share one
 * field inversion (PR #23738 "TL;DR", PR #23736 "Goal & lever"; S = 8 is the pages'
 * default, PR #23738 "What landed here"), the pairs of each bucket are reduced level
 * by level (the pair-tree of PR #23520, "Summary"), and the bucket sums are combined
 * per window by a running sum and across windows by doubling. The curve is the one
 * barretenberg uses; the pages do not name it, so its constants are EIP-196's.
 * Before windowing, each scalar is split by the curve's endomorphism phi(x, y) =
 * (beta x, y) = lambda (x, y) into s = k1 + k2 lambda (mod r) with |k1|, |k2| < 2^127
 * (GLV; not on the pages), so the windows run over 2n points of 127-bit scalars.
 *
 * Data formats (all little-endian):
 *   - a field element is eight 32-bit words holding x * 2^256 mod p (Montgomery
 *     form), fully reduced (< p);
 *   - a point is msm_g1_affine {x, y}, 64 bytes; the point at infinity is (0, 0);
 *   - a scalar is eight 32-bit words holding an integer below 2^256 (not Montgomery).
 *
 * Every call validates its arguments before touching the GPU. Return codes are the
 * MSM_* values below; msm_last_error() gives the calling thread's last message.
 * Device pointers are the caller's; the library never frees them.
 */
#ifndef MSM_H
#define MSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct msm_g1_affine {
  uint32_t x[8];
  uint32_t y[8];
} msm_g1_affine;

typedef struct msm_ctx msm_ctx;

enum {
  MSM_OK = 0,
  MSM_ERR_ARG = -1,        /* bad pointer, alignment, size, c, S or sched; workspace too small */
  MSM_ERR_HIP = -2,        /* a HIP runtime call or kernel launch failed */
  MSM_ERR_OOM = -3,        /* device or pinned host allocation failed */
  MSM_ERR_RANGE = -4,      /* internal: a GLV half-scalar came out >= 2^127 (not expected) */
  MSM_ERR_OFF_CURVE = -5   /* verify = 1 only: an input point or the result is not on the curve */
};

/* Accumulate schedules (the sched argument of msm_run). */
enum {
  MSM_SCHED_PAIR_TREE = 0, /* level 0 of a per-bucket pair tree, S pairs per lane */
  MSM_SCHED_WALKER = 1     /* stream walker: S slots per lane walk equal chunks of the lists */
};

/* Scalar forms (msm_ctx_set_scalar_form). */
enum {
  MSM_SCALARS_INTEGER = 0,   /* s_i as 256-bit little-endian integers (any value; used mod r) */
  MSM_SCALARS_MONTGOMERY = 1 /* s_i as Montgomery-form F_r elements, x * 2^256 mod r */
};

/* Largest n accepted. Bucket lists are indexed with 32-bit offsets, so in addition
 * 2 n ceil(128 / c) must stay below 2^32 (every c >= 5 allows MSM_MAX_N). */
#define MSM_MAX_N ((size_t)1 << 26)

/* Library version, major * 10000 + minor * 100 + patch. */
int msm_version(void);

/* Message describing the calling thread's most recent error ("" if none). */
const char* msm_last_error(void);

/*
 * Context: binds a device and owns a growable workspace, a pinned host buffer for the
 * one mid-pipeline read-back, a small device result buffer and the event that orders
 * its calls. Calls on one context must not be made from several host threads at once.
 * Returns MSM_ERR_ARG for a bad device or NULL out, MSM_ERR_OOM if the pinned or
 * device buffers cannot be allocated.
 */
int msm_ctx_create(int device, msm_ctx** out);
void msm_ctx_destroy(msm_ctx* ctx);

/*
 * Device workspace bytes msm_run needs for n points with window c and S slots (the
 * analogue of the pages' estimateMem, PR #23520 "Summary"); the same size serves both
 * schedules. S changes it only for small n, where the stream walker's slot state is the
 * larger part. Returns 0 for invalid n, c or S.
 */
size_t msm_workspace_bytes(size_t n, int c, int S);

/*
 * Q = sum_i s_i * P_i on `stream` (a hipStream_t; NULL is the null stream).
 *   d_points   device, n msm_g1_affine, 16-byte aligned; every point on the curve or
 *              (0, 0). Without verify the library does not check curve membership.
 *   d_scalars  device, n * 8 uint32 words, 16-byte aligned; any 256-bit integers
 *              (reduced mod r on the device).
 *   n          0 .. MSM_MAX_N with 2 n ceil(128 / c) < 2^32; n = 0 gives the point
 *              at infinity.
 *   c          window width in bits, 1 .. 16; W = ceil(128 / c) windows of signed
 *              digits in [-2^(c-1), 2^(c-1)] over the 2n half-scalars (2^(c-1)
 *              buckets per window, -P is free).
 *   S          affine additions sharing one field inversion: 4, 8, 16 or 32
 *              (PR #23738 "TL;DR"; PR #23736 "Goal & lever").
 *   sched      MSM_SCHED_PAIR_TREE: each lane adds S pairs of one or more bucket lists
 *              at pair-tree level 0 (PR #23520 "Summary"); deeper levels follow.
 *              MSM_SCHED_WALKER: each lane owns S slots, each walking an equal chunk of
 *              the sorted lists with one batched inversion per step; finished buckets
 *              are flushed and chunk-boundary partial sums combined afterwards
 *              (PR #23736 "Change"; PR #23738 "What would actually win").
 *   verify     0 or 1. With 1, every input point is checked on the device (coordinates
 *              below p, y^2 = x^3 + 3, or (0, 0)) and so is the result, the failure
 *              signal of PR #23736 ("Correctness-harness fix"); the call then waits
 *              for the stream to read the result's flag. An off-curve input returns
 *              MSM_ERR_OFF_CURVE before the accumulate is enqueued (d_out is not
 *              written); an off-curve result returns it after d_out is written.
 *   d_workspace device scratch of msm_workspace_bytes(n, c, S) bytes (256-byte
 *              aligned), or NULL to use the context's own (grown on demand).
 *   workspace_bytes  size of d_workspace (ignored when it is NULL); the library
 *              checks it against msm_workspace_bytes before any launch.
 *   d_out      device, one msm_g1_affine: Q in affine Montgomery form, (0, 0) if
 *              Q is the point at infinity.
 * The call enqueues the decompose/count/sort kernels, then blocks once on `stream`
 * to read back a small plan (largest bucket, split range flag), then enqueues the
 * accumulate, reduction and combine kernels and returns; d_out is valid once the
 * stream reaches that point. Consecutive calls on one context are ordered on the
 * device even when they use different streams (each call waits for the previous
 * call's last kernel), so the context's workspace is never shared by two calls in
 * flight. Points must lie in the prime-order group (every BN254 G1 point does: the
 * cofactor is 1). MSM_ERR_RANGE only if the split's bound failed, which the
 * constants rule out (nothing further is enqueued then).
 */
int msm_run(msm_ctx* ctx, const msm_g1_affine* d_points, const uint32_t* d_scalars, size_t n,
            int c, int S, int sched, int verify, void* d_workspace, size_t workspace_bytes,
            void* stream, msm_g1_affine* d_out);

/*
 * msm_run without allocation, for callers that cannot allocate device memory while
 * they run (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments and results as msm_run with d_workspace = NULL, except
 * that the workspace is a fixed device array of MSM_NOALLOC_MAX_BYTES built into the
 * library (one copy per GPU, held until the process ends) instead of the context's
 * growable one, and the context's phase timing is not recorded. The call allocates
 * nothing: no hipMalloc, no pinned memory, no events (the context made those when it
 * was created). Limits: msm_workspace_bytes(n, c, S) must not exceed
 * MSM_NOALLOC_MAX_BYTES, else MSM_ERR_ARG (c = 8 or 13 allows n up to about 10,000;
 * c = 16 needs more than the array at any n). All calls on one GPU share the one
 * array: calls that overlap on a GPU (from two contexts, or two host threads) race
 * and give wrong results; calls on one context are ordered as for msm_run. Like
 * msm_run it blocks once on `stream` for the plan, so it cannot itself be captured
 * into a graph. MSM_ERR_HIP if the array's address could not be looked up.
 */
#define MSM_NOALLOC_MAX_BYTES ((size_t)64 << 20)
int msm_run_noalloc(msm_ctx* ctx, const msm_g1_affine* d_points, const uint32_t* d_scalars,
                    size_t n, int c, int S, int sched, int verify, void* stream,
                    msm_g1_affine* d_out);

/*
 * Synchronous convenience form, the shape msm(points_affine, scalars, n, c) -> point:
 * device inputs, result written to host memory h_out. Uses a per-device default
 * context (created on first use), S = 8, the pair-tree schedule, no verify and the
 * null stream; the result travels through a small device buffer the context owns,
 * so a call allocates nothing after the context's workspace has grown to n.
 * Calls from several host threads are serialized.
 */
int msm(const msm_g1_affine* d_points, const uint32_t* d_scalars, size_t n, int c,
        msm_g1_affine* h_out);

/*
 * d_out[i] = k_i * G for the BN254 generator G = (1, 2), in the point format above.
 * d_k: device, n * 8 uint32 words (any 256-bit integers). Asynchronous on `stream`.
 * Builds synthetic inputs of the pages' kind: independent points r_i * G
 * (PR #23736, "Correctness-harness fix").
 */
int msm_g1_from_scalars(const uint32_t* d_k, size_t n, msm_g1_affine* d_out, void* stream);

/*
 * Pair-tree schedule: the first `levels` levels of every bucket's pair tree use the
 * batched affine adder (S adds per lane share one inversion); the remaining levels
 * use XYZZ coordinates, one addition per lane and no inversion, which shortens the
 * deep levels where few pairs are left. -1 makes every level affine. Default 1.
 * Returns MSM_ERR_ARG for a NULL ctx or levels outside -1 .. 32.
 */
int msm_ctx_set_affine_levels(msm_ctx* ctx, int levels);

/*
 * Where the stream walker (MSM_SCHED_WALKER) keeps each slot's accumulator (acc_x,
 * acc_y) and current bucket: 1 (default) in a device buffer, word-major over slots, as
 * PR #23738 ("What would actually win") proposes; 0 in per-lane arrays that the compiler
 * places in private memory, as the pages' walker does (PR #23738 "TL;DR"). The batch's
 * prefix products are private either way. The result does not depend on it. Returns
 * MSM_ERR_ARG for a NULL ctx or a value other than 0 or 1.
 */
int msm_ctx_set_walker_state(msm_ctx* ctx, int device_state);

/*
 * Where the batched-affine pair-tree level kernel keeps each lane's slot state:
 * store 0 (default) puts the S prefix products in per-lane arrays that the compiler
 * places in private memory; 1 puts them in the block's LDS (S * 32 bytes per lane, one
 * wavefront per block); adding 2 also caches each slot's denominator next to its prefix
 * (the dx cache of PR #23520 "Summary"), so the backward pass does not form it again;
 * 4 keeps only every fourth prefix (in private memory) and rebuilds the other three and
 * the denominators in registers in the backward pass (3 more products per 4 slots for
 * a quarter of the state). The result does not depend on it. Returns MSM_ERR_ARG for a
 * NULL ctx or store outside 0 .. 4.
 */
int msm_ctx_set_prefix_store(msm_ctx* ctx, int store);

/*
 * How the context's runs read the scalars: MSM_SCALARS_INTEGER (default) takes each
 * s_i as a 256-bit integer, reduced mod r; MSM_SCALARS_MONTGOMERY takes s_i as the
 * Montgomery form x * 2^256 mod r of the scalar x (how a prover's F_r code keeps
 * scalars; the pages' scalars enter as field elements of barretenberg's "bb/msm") and
 * converts it on the device (x = s_i * 2^-256 mod r, for any 256-bit s_i) before the
 * GLV split. The layout is the same: eight little-endian 32-bit words per scalar.
 * Returns MSM_ERR_ARG for a NULL ctx or another value.
 */
int msm_ctx_set_scalar_form(msm_ctx* ctx, int form);

/*
 * Phase timing. msm_ctx_set_timing(ctx, level) makes msm_run record HIP events on its
 * stream: level 1 brackets only the batched-affine accumulate kernel launches and the
 * window-combine kernel (what the rooflines of those kernels need, at the least cost to
 * the rest of the pipeline); level 2 also brackets each phase: sort (count, scan, scatter), accumulate (bucket init and
 * all pair-tree levels, each XYZZ level kernel on its own), reduce (running sums) and
 * final (window combine); level 0 turns timing off. Each event pair costs the stream
 * a few microseconds. msm_ctx_timing_read waits for the events recorded since the
 * last read, sums them into *out and resets. Returns MSM_ERR_ARG for NULL arguments
 * or a level outside 0 .. 2.
 */
typedef struct msm_timing {
  double sort_ms;          /* decompose, histogram, scans, scatter (incl. the read-back) */
  double accumulate_ms;    /* bucket init + all pair-tree levels (scans included) */
  double level_kernel_ms;  /* the pair-tree level kernels alone */
  double reduce_ms;        /* running-sum segments + per-window trees */
  double final_ms;         /* window combine and conversion to affine */
  int runs;                /* msm_run calls summed */
  int level_launches;      /* level kernel launches summed */
  uint64_t level_pairs;    /* affine additions done by those launches */
  uint64_t level_lanes;    /* lanes that ran them (one inversion each) */
  double xyzz_level_ms;    /* pair-tree levels done in XYZZ coordinates */
} msm_timing;

int msm_ctx_set_timing(msm_ctx* ctx, int enable);
int msm_ctx_timing_read(msm_ctx* ctx, msm_timing* out);

/*
 * Test hooks (the same device code as the MSM, exposed for unit tests). All take
 * device pointers to n field elements of eight words each (Montgomery form, < p) and
 * run asynchronously on `stream`.
 *
 * msm_test_fp_mul / _sqr / _add / _sub: d_out = a*b, a^2, a+b, a-b (Montgomery
 * products a*b*2^-256 mod p for mul and sqr).
 * msm_test_fp_inv: d_out = a^-1 (the Montgomery form of the inverse) by the binary-GCD
 * inverse every kernel uses; 0 gives 0.
 *
 * msm_test_fp: the same operations by number, plus conversions and the inverse's
 * parts: op 0 a*b, 1 a+b, 2 a-b, 3 a^2, 4 a^-1 (0 -> 0), 5 to Montgomery (a * 2^256),
 * 6 from Montgomery (a * 2^-256), 7 Fermat's a^(p-2) alone, 8 the binary-GCD inverse
 * with no special case for 0 (its own fallback handles it). d_b unused for unary ops.
 *
 * msm_test_batched_add: d_out[i] = d_a[i] + d_b[i] for n affine points, computed by
 * the batched-affine adder with S slots per lane (one inversion per S sums, PR #23520
 * "Summary"); every special case (infinity, doubling, P + (-P)) is allowed.
 *
 * msm_test_glv: the scalar split of msm_run for n scalars (8 words each, any
 * 256-bit value): d_halfs[i] = |k1| and d_halfs[n + i] = |k2| of scalar i, four
 * words each with the sign in bit 127, where s = k1 + k2 lambda (mod r).
 * d_halfs holds 2 n * 4 words.
 *
 * msm_test_row: the row form of the field arithmetic that the window combine's runs of
 * doublings use (one product spread over the 16 lanes of a DPP row, four products per
 * wavefront). op 0 a*b, 1 a+b, 2 a-b on n elements (8 words each, fully reduced
 * Montgomery form, like msm_test_fp); op 3 d_out[i] = 2^d * d_a[i] for n XYZZ points (32
 * words each: X, Y, ZZ, ZZZ, fully reduced; d <= 4096) by runs of doublings in row form,
 * op 4 the same by the quad runs; ops 5 and 6 are a latency probe on one wavefront
 * (n = 4): x <- x * b, d times, for the four elements of d_a and d_b, in row form (5) or
 * with the per-lane product (6), the four results to d_out; op 7 d_out[i] = d_a[i] +
 * d_b[i] and op 8 d_out[i] = 2 * d_a[i] for n XYZZ points by the row-form point
 * arithmetic of the window combine (any inputs: infinity, equal and opposite points);
 * op 9 d_out[i] (16 words: x, y, infinity as (0, 0)) = d_a[i] in affine coordinates by
 * the combine's final conversion. d_b is used by ops 0..2 and 5..7 only.
 *
 * msm_test_issue_rate: an instruction-rate probe of the device (not a field
 * operation): `blocks` blocks of 256 lanes each run `iters` rounds of 16 independent
 * chains of one instruction class, op 0 the 32x32->64-bit multiply-add that the
 * Montgomery product is made of (v_mad_u64_u32), op 1 a 32-bit add, op 2 a 32-bit add
 * with carry in and out (the field add/sub chains); lane i writes a fold of its chains
 * to d_out[i] (blocks * 256 words). Timing it with events gives the sustained issue rate
 * of the class, which sets the peak of the integer roofline.
 *
 * Errors: MSM_ERR_ARG for an unknown op or S, n > MSM_MAX_N, NULL or misaligned
 * pointers with n > 0 (for the probe: blocks outside 1 .. 2^20, iters = 0 or a NULL
 * d_out); MSM_ERR_HIP if the launch fails.
 */
int msm_test_fp(int op, const uint32_t* d_a, const uint32_t* d_b, uint32_t* d_out, size_t n,
                void* stream);
int msm_test_fp_mul(const uint32_t* d_a, const uint32_t* d_b, uint32_t* d_out, size_t n, void* stream);
int msm_test_fp_sqr(const uint32_t* d_a, uint32_t* d_out, size_t n, void* stream);
int msm_test_fp_add(const uint32_t* d_a, const uint32_t* d_b, uint32_t* d_out, size_t n, void* stream);
int msm_test_fp_sub(const uint32_t* d_a, const uint32_t* d_b, uint32_t* d_out, size_t n, void* stream);
int msm_test_fp_inv(const uint32_t* d_a, uint32_t* d_out, size_t n, void* stream);
int msm_test_glv(const uint32_t* d_scalars, size_t n, uint32_t* d_halfs, void* stream);
int msm_test_row(int op, const uint32_t* d_a, const uint32_t* d_b, uint32_t* d_out, size_t n,
                 uint32_t d, void* stream);
int msm_test_issue_rate(int op, uint32_t blocks, uint32_t iters, uint32_t* d_out, void* stream);
int msm_test_batched_add(const msm_g1_affine* d_a, const msm_g1_affine* d_b,
                         msm_g1_affine* d_out, size_t n, int S, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSM_H */
