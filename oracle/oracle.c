/*
 * Oracle: a plain CPU reference for the BN254 G1 multi-scalar multiplication
 *     Q = sum_i s_i * P_i.
 *
 * TEST INFRASTRUCTURE ONLY. The product library never links, loads or calls this
 * file; only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg do.
 * It shares no code, header, table or constant generator with the GPU library.
 *
 * Source of the method: aztec-packages PR #23738 / #23736 / #23520 ("bb/msm"):
 * a Pippenger bucket MSM (bucket lists sorted by bucket, window c = 13 at
 * n = 2^16, PR #23520 "Measurements"), checked against an independent
 * implementation for an on-curve, bit-identical result (PR #23736,
 * "Correctness-harness fix"). The pages name no curve; this is BN254 / alt_bn128
 * (the curve barretenberg uses; constants from EIP-196).
 *
 * Deliberately different from the GPU library in every layer:
 *   - field elements are 4 x 64-bit limbs multiplied with unsigned __int128
 *     (the GPU uses 8 x 32-bit limbs), always kept fully reduced;
 *   - points are Jacobian (X:Y:Z), x = X/Z^2, y = Y/Z^3, with the textbook
 *     formulas (Hankerson-Menezes-Vanstone, "Guide to ECC", ch. 3), Z = 0 = infinity;
 *     the mixed case is the general addition with Z2 = 1 (the GPU uses batched
 *     affine additions and XYZZ coordinates);
 *   - inversion is Fermat, x^(p-2);
 *   - Pippenger is the plain one: one thread per window, every point added into
 *     its bucket one by one, a sequential running sum, Horner over windows.
 *
 * Interchange format (shared with the tests): a coordinate is x * 2^256 mod p as
 * little-endian words (8 x u32 == 4 x u64 on little-endian hosts); a point is
 * x then y (64 bytes); (0,0) is the point at infinity. Scalars are 256-bit
 * little-endian integers.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef unsigned __int128 u128;

typedef struct { uint64_t v[4]; } fe;          /* Montgomery form, always < p */
typedef struct { fe x, y; } aff;               /* affine; infinity flagged separately */
typedef struct { fe X, Y, Z; } jac;            /* Jacobian; Z == 0 is infinity */

enum { ORACLE_OK = 0, ORACLE_ERR_ARG = -1, ORACLE_ERR_POINT = -5, ORACLE_ERR_RANGE = -4 };

/* EIP-196 base-field prime p, as 4 little-endian 64-bit words. */
static const uint64_t PM[4] = {0x3c208c16d87cfd47ULL, 0x97816a916871ca8dULL,
                               0xb85045b68181585dULL, 0x30644e72e131a029ULL};
/* -p^{-1} mod 2^64 (the Montgomery constant for 64-bit words). */
static const uint64_t PINV = 0x87d20782e4866389ULL;
/* 2^512 mod p (converts an integer into Montgomery form). */
static const fe R2 = {{0xf32cfc5b538afa89ULL, 0xb5e71911d44501fbULL, 0x47ab1eff0a417ff6ULL,
                       0x06d89f71cab8351fULL}};

/* ------------------------------------------------------------------ field F_p */
static int fe_is_zero(const fe *a) { return (a->v[0] | a->v[1] | a->v[2] | a->v[3]) == 0; }

static int fe_eq(const fe *a, const fe *b) { return memcmp(a->v, b->v, sizeof a->v) == 0; }

/* t >= p ? (t given as 4 words) */
static int geq_p(const uint64_t t[4]) {
    for (int i = 3; i >= 0; i--) {
        if (t[i] > PM[i]) return 1;
        if (t[i] < PM[i]) return 0;
    }
    return 1;
}

static void sub_p(uint64_t t[4]) {
    u128 borrow = 0;
    for (int i = 0; i < 4; i++) {
        u128 d = (u128)t[i] - PM[i] - borrow;
        t[i] = (uint64_t)d;
        borrow = (d >> 64) & 1;
    }
}

static void fe_add(fe *r, const fe *a, const fe *b) {
    uint64_t t[4];
    u128 c = 0;
    for (int i = 0; i < 4; i++) {
        c += (u128)a->v[i] + b->v[i];
        t[i] = (uint64_t)c;
        c >>= 64;
    }
    /* a, b < p < 2^254, so the sum has no carry out of 256 bits */
    if (geq_p(t)) sub_p(t);
    memcpy(r->v, t, sizeof t);
}

static void fe_sub(fe *r, const fe *a, const fe *b) {
    uint64_t t[4];
    u128 borrow = 0;
    for (int i = 0; i < 4; i++) {
        u128 d = (u128)a->v[i] - b->v[i] - borrow;
        t[i] = (uint64_t)d;
        borrow = (d >> 64) & 1;
    }
    if (borrow) { /* a < b: add p back */
        u128 c = 0;
        for (int i = 0; i < 4; i++) {
            c += (u128)t[i] + PM[i];
            t[i] = (uint64_t)c;
            c >>= 64;
        }
    }
    memcpy(r->v, t, sizeof t);
}

/* Montgomery product a*b*2^-256 mod p, coarsely integrated operand scanning. */
static void fe_mul(fe *r, const fe *a, const fe *b) {
    uint64_t t[5] = {0, 0, 0, 0, 0};
    for (int i = 0; i < 4; i++) {
        uint64_t carry = 0;
        for (int j = 0; j < 4; j++) {
            u128 acc = (u128)a->v[j] * b->v[i] + t[j] + carry;
            t[j] = (uint64_t)acc;
            carry = (uint64_t)(acc >> 64);
        }
        u128 top = (u128)t[4] + carry;
        t[4] = (uint64_t)top;
        uint64_t t5 = (uint64_t)(top >> 64);

        uint64_t m = t[0] * PINV;
        u128 acc = (u128)m * PM[0] + t[0];
        carry = (uint64_t)(acc >> 64);
        for (int j = 1; j < 4; j++) {
            acc = (u128)m * PM[j] + t[j] + carry;
            t[j - 1] = (uint64_t)acc;
            carry = (uint64_t)(acc >> 64);
        }
        top = (u128)t[4] + carry;
        t[3] = (uint64_t)top;
        t[4] = t5 + (uint64_t)(top >> 64);
    }
    /* inputs < p give a result < 2p < 2^256, so t[4] is 0 here */
    if (t[4] || geq_p(t)) sub_p(t);
    memcpy(r->v, t, 4 * sizeof(uint64_t));
}

static void fe_sqr(fe *r, const fe *a) { fe_mul(r, a, a); }

static void fe_one(fe *r) { /* 2^256 mod p: Montgomery form of 1 */
    fe plain = {{1, 0, 0, 0}};
    fe_mul(r, &plain, &R2);
}

/* x^e for a 256-bit exponent, left-to-right square and multiply. */
static void fe_pow(fe *r, const fe *x, const uint64_t e[4]) {
    fe acc;
    fe_one(&acc);
    for (int i = 255; i >= 0; i--) {
        fe_sqr(&acc, &acc);
        if ((e[i / 64] >> (i % 64)) & 1) fe_mul(&acc, &acc, x);
    }
    *r = acc;
}

/* Inverse by Fermat: x^(p-2). x must be non-zero. */
static void fe_inv(fe *r, const fe *x) {
    uint64_t e[4] = {PM[0] - 2, PM[1], PM[2], PM[3]}; /* p's low word is > 2 */
    fe_pow(r, x, e);
}

static void fe_small(fe *r, uint64_t k) { /* Montgomery form of a small integer */
    fe plain = {{k, 0, 0, 0}};
    fe_mul(r, &plain, &R2);
}

/* ------------------------------------------------------------------ curve (a = 0, b = 3) */
static void jac_set_inf(jac *r) { memset(r, 0, sizeof *r); }
static int jac_is_inf(const jac *a) { return fe_is_zero(&a->Z); }

static void jac_from_aff(jac *r, const aff *a, int inf) {
    if (inf) { jac_set_inf(r); return; }
    r->X = a->x;
    r->Y = a->y;
    fe_one(&r->Z);
}

/* 2P: S = 4XY^2, M = 3X^2, X3 = M^2 - 2S, Y3 = M(S - X3) - 8Y^4, Z3 = 2YZ. */
static void jac_dbl(jac *r, const jac *p) {
    if (jac_is_inf(p) || fe_is_zero(&p->Y)) { jac_set_inf(r); return; }
    fe yy, s, m, t, x3, y3, z3, yyyy;
    fe_sqr(&yy, &p->Y);
    fe_mul(&s, &p->X, &yy);
    fe_add(&s, &s, &s);
    fe_add(&s, &s, &s);                     /* S = 4 X Y^2 */
    fe_sqr(&m, &p->X);
    fe_add(&t, &m, &m);
    fe_add(&m, &t, &m);                     /* M = 3 X^2 */
    fe_sqr(&x3, &m);
    fe_sub(&x3, &x3, &s);
    fe_sub(&x3, &x3, &s);                   /* X3 = M^2 - 2S */
    fe_sqr(&yyyy, &yy);
    fe_add(&yyyy, &yyyy, &yyyy);
    fe_add(&yyyy, &yyyy, &yyyy);
    fe_add(&yyyy, &yyyy, &yyyy);            /* 8 Y^4 */
    fe_sub(&t, &s, &x3);
    fe_mul(&y3, &m, &t);
    fe_sub(&y3, &y3, &yyyy);                /* Y3 = M (S - X3) - 8 Y^4 */
    fe_mul(&z3, &p->Y, &p->Z);
    fe_add(&z3, &z3, &z3);                  /* Z3 = 2 Y Z */
    r->X = x3;
    r->Y = y3;
    r->Z = z3;
}

/* P1 + P2, general Jacobian addition with every special case. */
static void jac_add(jac *r, const jac *p1, const jac *p2) {
    if (jac_is_inf(p1)) { *r = *p2; return; }
    if (jac_is_inf(p2)) { *r = *p1; return; }
    fe z1z1, z2z2, u1, u2, s1, s2, h, rr, t;
    fe_sqr(&z1z1, &p1->Z);
    fe_sqr(&z2z2, &p2->Z);
    fe_mul(&u1, &p1->X, &z2z2);             /* U1 = X1 Z2^2 */
    fe_mul(&u2, &p2->X, &z1z1);             /* U2 = X2 Z1^2 */
    fe_mul(&t, &z2z2, &p2->Z);
    fe_mul(&s1, &p1->Y, &t);                /* S1 = Y1 Z2^3 */
    fe_mul(&t, &z1z1, &p1->Z);
    fe_mul(&s2, &p2->Y, &t);                /* S2 = Y2 Z1^3 */
    fe_sub(&h, &u2, &u1);                   /* H = U2 - U1 */
    fe_sub(&rr, &s2, &s1);                  /* R = S2 - S1 */
    if (fe_is_zero(&h)) {
        if (fe_is_zero(&rr)) { jac_dbl(r, p1); return; } /* same point */
        jac_set_inf(r);                                   /* P + (-P) */
        return;
    }
    fe hh, hhh, u1hh, x3, y3, z3;
    fe_sqr(&hh, &h);
    fe_mul(&hhh, &hh, &h);
    fe_mul(&u1hh, &u1, &hh);
    fe_sqr(&x3, &rr);
    fe_sub(&x3, &x3, &hhh);
    fe_sub(&x3, &x3, &u1hh);
    fe_sub(&x3, &x3, &u1hh);                /* X3 = R^2 - H^3 - 2 U1 H^2 */
    fe_sub(&t, &u1hh, &x3);
    fe_mul(&y3, &rr, &t);
    fe_mul(&t, &s1, &hhh);
    fe_sub(&y3, &y3, &t);                   /* Y3 = R (U1 H^2 - X3) - S1 H^3 */
    fe_mul(&z3, &p1->Z, &p2->Z);
    fe_mul(&z3, &z3, &h);                   /* Z3 = Z1 Z2 H */
    r->X = x3;
    r->Y = y3;
    r->Z = z3;
}

/* Jacobian -> affine; returns 1 for infinity. */
static int jac_to_aff(aff *r, const jac *p) {
    if (jac_is_inf(p)) { memset(r, 0, sizeof *r); return 1; }
    fe zi, zi2, zi3;
    fe_inv(&zi, &p->Z);
    fe_sqr(&zi2, &zi);
    fe_mul(&zi3, &zi2, &zi);
    fe_mul(&r->x, &p->X, &zi2);
    fe_mul(&r->y, &p->Y, &zi3);
    return 0;
}

/* ------------------------------------------------------------------ interchange */
static int load_point(aff *a, const uint32_t w[16], int *inf) {
    memcpy(a->x.v, w, 32);
    memcpy(a->y.v, w + 8, 32);
    if (fe_is_zero(&a->x) && fe_is_zero(&a->y)) { *inf = 1; return ORACLE_OK; }
    *inf = 0;
    if (geq_p(a->x.v) || geq_p(a->y.v)) return ORACLE_ERR_POINT;
    fe lhs, rhs, three;
    fe_sqr(&lhs, &a->y);
    fe_sqr(&rhs, &a->x);
    fe_mul(&rhs, &rhs, &a->x);
    fe_small(&three, 3);
    fe_add(&rhs, &rhs, &three);
    return fe_eq(&lhs, &rhs) ? ORACLE_OK : ORACLE_ERR_POINT;
}

static void store_jac(uint32_t w[16], const jac *p) {
    aff a;
    jac_to_aff(&a, p);
    memcpy(w, a.x.v, 32);
    memcpy(w + 8, a.y.v, 32);
}

static int scalar_bit(const uint32_t k[8], int i) { return i < 256 ? (k[i >> 5] >> (i & 31)) & 1 : 0; }

static void jac_scalar_mul(jac *r, const jac *p, const uint32_t k[8]) {
    jac acc;
    jac_set_inf(&acc);
    for (int i = 255; i >= 0; i--) {
        jac_dbl(&acc, &acc);
        if (scalar_bit(k, i)) jac_add(&acc, &acc, p);
    }
    *r = acc;
}

/* ------------------------------------------------------------------ exports: field */
/* Batched field operations on Montgomery-form inputs, for pinning against Python ints.
 * op: 0 mul, 1 add, 2 sub, 3 sqr, 4 inv (0 -> 0), 5 to Montgomery, 6 from Montgomery. */
int oracle_fp_op(int op, const uint64_t *a, const uint64_t *b, uint64_t *out, size_t n) {
    for (size_t i = 0; i < n; i++) {
        fe x, y, z;
        memcpy(x.v, a + 4 * i, 32);
        if (b) memcpy(y.v, b + 4 * i, 32);
        switch (op) {
        case 0: fe_mul(&z, &x, &y); break;
        case 1: fe_add(&z, &x, &y); break;
        case 2: fe_sub(&z, &x, &y); break;
        case 3: fe_sqr(&z, &x); break;
        case 4: if (fe_is_zero(&x)) memset(&z, 0, sizeof z); else fe_inv(&z, &x); break;
        case 5: fe_mul(&z, &x, &R2); break;
        case 6: { fe one = {{1, 0, 0, 0}}; fe_mul(&z, &x, &one); } break;
        default: return ORACLE_ERR_ARG;
        }
        memcpy(out + 4 * i, z.v, 32);
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ exports: curve */
int oracle_g1_on_curve(const uint32_t pt[16]) {
    aff a;
    int inf;
    return load_point(&a, pt, &inf) == ORACLE_OK;
}

/* out = k * pt by MSB-first double-and-add. */
int oracle_g1_scalar_mul(const uint32_t pt[16], const uint32_t k[8], uint32_t out[16]) {
    aff a;
    int inf, rc = load_point(&a, pt, &inf);
    if (rc) return rc;
    jac p, q;
    jac_from_aff(&p, &a, inf);
    jac_scalar_mul(&q, &p, k);
    store_jac(out, &q);
    return ORACLE_OK;
}

/* out = p1 + p2 (affine interchange in and out). */
int oracle_g1_add(const uint32_t p1[16], const uint32_t p2[16], uint32_t out[16]) {
    aff a, b;
    int ia, ib, rc;
    if ((rc = load_point(&a, p1, &ia)) || (rc = load_point(&b, p2, &ib))) return rc;
    jac ja, jb, jr;
    jac_from_aff(&ja, &a, ia);
    jac_from_aff(&jb, &b, ib);
    jac_add(&jr, &ja, &jb);
    store_jac(out, &jr);
    return ORACLE_OK;
}

/* ---- fixed-base points k_i * G, k = sum_j byte_j 256^j, G_j = 256^j G ---- */
static aff comb_tab[32][256];  /* comb_tab[j][d] = d * 256^j * G (d >= 1) */
static pthread_once_t comb_once = PTHREAD_ONCE_INIT;

static void comb_build(void) {
    jac base, acc;
    fe_one(&base.Z);
    fe_small(&base.X, 1);
    fe_small(&base.Y, 2);                   /* G = (1, 2) */
    for (int j = 0; j < 32; j++) {
        acc = base;
        for (int d = 1; d < 256; d++) {
            jac_to_aff(&comb_tab[j][d], &acc);
            jac_add(&acc, &acc, &base);
        }
        for (int t = 0; t < 8; t++) jac_dbl(&base, &base);
    }
}

typedef struct {
    const uint32_t *k;
    uint32_t *out;
    size_t n;
    size_t next;
    pthread_mutex_t mu;
} gen_job;

static void *gen_worker(void *arg) {
    gen_job *job = (gen_job *)arg;
    for (;;) {
        pthread_mutex_lock(&job->mu);
        size_t lo = job->next;
        job->next += 256;
        pthread_mutex_unlock(&job->mu);
        if (lo >= job->n) break;
        size_t hi = lo + 256 < job->n ? lo + 256 : job->n;
        for (size_t i = lo; i < hi; i++) {
            const uint8_t *bytes = (const uint8_t *)(job->k + 8 * i);
            jac acc, t;
            jac_set_inf(&acc);
            for (int j = 0; j < 32; j++) {
                if (!bytes[j]) continue;
                jac_from_aff(&t, &comb_tab[j][bytes[j]], 0);
                jac_add(&acc, &acc, &t);
            }
            store_jac(job->out + 16 * i, &acc);
        }
    }
    return NULL;
}

static int clamp_threads(int threads) {
    if (threads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        threads = c > 0 ? (int)c : 1;
    }
    return threads > 256 ? 256 : threads;
}

int oracle_threads_default(void) { return clamp_threads(0); }

/* out[i] = k[i] * G for n 256-bit scalars (little-endian u32 words). */
int oracle_g1_from_scalars(const uint32_t *k, size_t n, uint32_t *out, int threads) {
    pthread_once(&comb_once, comb_build);
    gen_job job = {k, out, n, 0, PTHREAD_MUTEX_INITIALIZER};
    threads = clamp_threads(threads);
    pthread_t tid[256];
    for (int t = 0; t < threads; t++) pthread_create(&tid[t], NULL, gen_worker, &job);
    for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ exports: MSM */
/* Definition written out: Q = sum_i s_i * P_i, each term by double-and-add. */
int oracle_msm_naive(const uint32_t *points, const uint32_t *scalars, size_t n, uint32_t out[16]) {
    jac acc, p, t;
    jac_set_inf(&acc);
    for (size_t i = 0; i < n; i++) {
        aff a;
        int inf, rc = load_point(&a, points + 16 * i, &inf);
        if (rc) return rc;
        jac_from_aff(&p, &a, inf);
        jac_scalar_mul(&t, &p, scalars + 8 * i);
        jac_add(&acc, &acc, &t);
    }
    store_jac(out, &acc);
    return ORACLE_OK;
}

typedef struct {
    const aff *pts;
    const uint8_t *inf;
    const uint32_t *sc;
    size_t n;
    int c, nwin;
    jac *win;
    jac *bucket_out;   /* optional: per-window bucket sums, nwin * 2^c entries */
    int next;
    pthread_mutex_t mu;
} msm_job;

static uint32_t digit(const uint32_t k[8], int j, int c) {
    uint32_t d = 0;
    for (int b = 0; b < c; b++) d |= (uint32_t)scalar_bit(k, j * c + b) << b;
    return d;
}

static void *msm_worker(void *arg) {
    msm_job *job = (msm_job *)arg;
    size_t nb = (size_t)1 << job->c;
    jac *bucket = (jac *)malloc(nb * sizeof(jac));
    for (;;) {
        pthread_mutex_lock(&job->mu);
        int j = job->next++;
        pthread_mutex_unlock(&job->mu);
        if (j >= job->nwin) break;
        for (size_t b = 0; b < nb; b++) jac_set_inf(&bucket[b]);
        for (size_t i = 0; i < job->n; i++) {
            uint32_t d = digit(job->sc + 8 * i, j, job->c);
            if (!d || job->inf[i]) continue;
            jac p;
            jac_from_aff(&p, &job->pts[i], 0);
            jac_add(&bucket[d], &bucket[d], &p);
        }
        if (job->bucket_out) memcpy(job->bucket_out + (size_t)j * nb, bucket, nb * sizeof(jac));
        /* W_j = sum_b b * bucket[b] as a running sum from the top bucket down. */
        jac run, tot;
        jac_set_inf(&run);
        jac_set_inf(&tot);
        for (size_t b = nb - 1; b >= 1; b--) {
            jac_add(&run, &run, &bucket[b]);
            jac_add(&tot, &tot, &run);
        }
        job->win[j] = tot;
    }
    free(bucket);
    return NULL;
}

/* Pippenger with unsigned c-bit windows, W = ceil(254 / c). Scalars >= 2^(W c) are
 * rejected with ORACLE_ERR_RANGE. Optionally returns the window sums W_j (affine
 * interchange, nwin * 16 words) and the bucket sums (nwin * 2^c * 16 words). */
int oracle_msm_pippenger_ex(const uint32_t *points, const uint32_t *scalars, size_t n, int c,
                            int threads, uint32_t out[16], uint32_t *win_out,
                            uint32_t *bucket_out) {
    if (c < 1 || c > 16 || (n && (!points || !scalars)) || !out) return ORACLE_ERR_ARG;
    int nwin = (254 + c - 1) / c;
    for (size_t i = 0; i < n; i++)
        for (int b = nwin * c; b < 256; b++)
            if (scalar_bit(scalars + 8 * i, b)) return ORACLE_ERR_RANGE;
    aff *pts = (aff *)malloc((n ? n : 1) * sizeof(aff));
    uint8_t *inf = (uint8_t *)malloc(n ? n : 1);
    for (size_t i = 0; i < n; i++) {
        int is_inf;
        if (load_point(&pts[i], points + 16 * i, &is_inf)) {
            free(pts);
            free(inf);
            return ORACLE_ERR_POINT;
        }
        inf[i] = (uint8_t)is_inf;
    }
    jac *win = (jac *)malloc(nwin * sizeof(jac));
    size_t nb = (size_t)1 << c;
    jac *bk = bucket_out ? (jac *)malloc((size_t)nwin * nb * sizeof(jac)) : NULL;
    msm_job job = {pts, inf, scalars, n, c, nwin, win, bk, 0, PTHREAD_MUTEX_INITIALIZER};
    threads = clamp_threads(threads);
    if (threads > nwin) threads = nwin;
    pthread_t tid[256];
    for (int t = 0; t < threads; t++) pthread_create(&tid[t], NULL, msm_worker, &job);
    for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);

    /* Horner over windows: Q = W_{W-1}; Q = 2^c Q + W_j for j = W-2 .. 0. */
    jac q;
    jac_set_inf(&q);
    for (int j = nwin - 1; j >= 0; j--) {
        for (int t = 0; t < c; t++) jac_dbl(&q, &q);
        jac_add(&q, &q, &win[j]);
    }
    store_jac(out, &q);
    if (win_out)
        for (int j = 0; j < nwin; j++) store_jac(win_out + 16 * j, &win[j]);
    if (bk) {
        for (size_t e = 0; e < (size_t)nwin * nb; e++) store_jac(bucket_out + 16 * e, &bk[e]);
        free(bk);
    }
    free(win);
    free(pts);
    free(inf);
    return ORACLE_OK;
}

int oracle_msm_pippenger(const uint32_t *points, const uint32_t *scalars, size_t n, int c,
                         int threads, uint32_t out[16]) {
    return oracle_msm_pippenger_ex(points, scalars, n, c, threads, out, NULL, NULL);
}
