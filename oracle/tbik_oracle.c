/*
 * tbik_oracle.c -- CPU oracle for the tree-based invariant kernels (TBIK).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, scalar definition
 * that the GPU library is checked against.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant with the HIP library: every constant below is
 * derived here from its mathematical definition.
 *
 * Sources (the web pages the method is taken from):
 *  [TBIK]  "Deterministic Inference across Tensor Parallel Sizes That
 *          Eliminates Training-Inference Mismatch" (Zhang et al., summary
 *          page): Abstract; method details, "technical framework" and
 *          "key design" paragraphs.
 *  [ROUND] winzheng.jp article on rounding-location alignment (Ke, Cai,
 *          Wang): "the problem" section (bf16 keeps 7 mantissa bits) and
 *          "surgical fix: three nodes" section (RoPE, SwiGLU, residual
 *          RMSNorm keep fp32 intermediates, round to bf16 once at the output).
 *  [ISO]   nxmr.cn brief on SkyRL IsoExec: section 叁 (execution contract:
 *          fixed accumulation blocking; bit-level train/infer comparison).
 *  [ND]    note "01-推理阶段的非确定性", section 2 (the order of a parallel
 *          sum changes its value).
 *  [DT]    note "09｜分布式训练、数值稳定性与评测证据", section 2.1.1 (the
 *          second MLP matrix split by input rows: each device produces a
 *          partial output of full shape and the partials are added).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *  R1 the tree TREE(v_0..v_{n-1}): T = largest power of two <= 8 dividing n,
 *     G = n/T consecutive leaves per group, PAIR inside each group, then a
 *     perfect binary tree over the T group sums;
 *  R2 PAIR: repeatedly add neighbours (u0+u1, u2+u3, ...); an odd last
 *     element moves up one level unchanged;
 *  R3 GEMM leaves are 64-wide K blocks, accumulated from +0 in K order;
 *  R4 EXP / LOG are defined by the operation sequences written below
 *     (Cody-Waite reduction plus Taylor polynomials), not by a libm;
 *  R5 two-pass log-softmax with the exact row maximum;
 *  R11 a misaligned rounding location is eager bf16 arithmetic (below);
 *  R12 backward passes: derivatives of the forward definitions in fp32,
 *      token sums by TREE over 64-token leaves (below).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (x86-64 SSE,
 * round-to-nearest, no FTZ/DAZ), so every float operation is one IEEE
 * binary32 operation.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32                                                             */
/* [ROUND] "the problem": bf16 has the fp32 exponent and 7 stored mantissa   */
/* bits, so a bf16 value is the top 16 bits of an fp32 pattern.              */
/* ------------------------------------------------------------------------ */

static float f_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

OR_EXPORT float or_bf16_to_f32(uint16_t h) { return f_from_bits((uint32_t)h << 16); }

/* Round-to-nearest-even of an fp32 value to bf16.  Decided by comparing the
 * discarded 16 bits with one half of a bf16 unit, written out as a plain
 * case analysis.  NaN becomes a quiet NaN with the same sign. */
OR_EXPORT uint16_t or_f32_to_bf16(float f) {
    uint32_t u = bits_from_f(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
    uint32_t hi = u >> 16;          /* truncated result */
    uint32_t lo = u & 0xffffu;      /* discarded part   */
    if (lo > 0x8000u) hi += 1;                          /* above half: up   */
    else if (lo == 0x8000u && (hi & 1u)) hi += 1;       /* tie: to even     */
    return (uint16_t)hi;            /* a carry into the exponent is correct */
}

/* ------------------------------------------------------------------------ */
/* The tree (R1, R2).  [TBIK] Abstract: intra- and inter-GPU reduction       */
/* orders are aligned through one hierarchical binary tree; "technical      */
/* framework": each GPU reduces its shard locally, then a binary tree        */
/* combines the GPUs.                                                        */
/* ------------------------------------------------------------------------ */

OR_EXPORT int or_tree_T(int64_t n) {
    int T = 8;
    while (T > 1 && (n % T) != 0) T /= 2;
    return T;
}

/* PAIR over u[0..m-1], level by level, in place.  Returns +0 for m == 0. */
static float pair_inplace(float *u, int64_t m) {
    if (m == 0) return 0.0f;
    while (m > 1) {
        int64_t half = m / 2;
        for (int64_t i = 0; i < half; i++) u[i] = u[2 * i] + u[2 * i + 1];
        if (m % 2 == 1) {
            u[half] = u[m - 1];   /* odd element carried unchanged */
            m = half + 1;
        } else {
            m = half;
        }
    }
    return u[0];
}

OR_EXPORT float or_pair(const float *v, int64_t m, float *scratch) {
    memcpy(scratch, v, (size_t)m * sizeof(float));
    return pair_inplace(scratch, m);
}

/* Sum of group g (0 <= g < T) of TREE over n leaves. */
static float group_sum(const float *v, int64_t n, int g, float *scratch) {
    int T = or_tree_T(n);
    int64_t G = n / T;
    memcpy(scratch, v + (int64_t)g * G, (size_t)G * sizeof(float));
    return pair_inplace(scratch, G);
}

OR_EXPORT float or_tree(const float *v, int64_t n, float *scratch) {
    if (n == 0) return 0.0f;
    int T = or_tree_T(n);
    float top[8];
    for (int g = 0; g < T; g++) top[g] = group_sum(v, n, g, scratch);
    return pair_inplace(top, T);
}

/* TREE evaluated the way T/tp "GPUs" would: shard t owns groups
 * [t*T/tp, (t+1)*T/tp), reduces them to its shard node, and the tp shard
 * nodes are then combined by a binary tree.  shard_nodes may be NULL. */
OR_EXPORT float or_tree_sharded(const float *v, int64_t n, int tp, float *scratch,
                                float *shard_nodes) {
    if (n == 0) return 0.0f;
    int T = or_tree_T(n);
    int per = T / tp;
    float nodes[8];
    for (int t = 0; t < tp; t++) {
        float gs[8];
        for (int q = 0; q < per; q++) gs[q] = group_sum(v, n, t * per + q, scratch);
        nodes[t] = pair_inplace(gs, per);
        if (shard_nodes) shard_nodes[t] = nodes[t];
    }
    return pair_inplace(nodes, tp);
}

/* ------------------------------------------------------------------------ */
/* EXP and LOG (R4).  Only IEEE-rounded add, mul, fma, div and bit moves.    */
/* ------------------------------------------------------------------------ */

/* Constants, each defined here from mathematics:
 *   log2(e) rounded to fp32;
 *   ln2 split as hi + lo, hi = ln2 rounded to a multiple of 2^-16 (so k*hi
 *   is exact for |k| < 2^8), lo = ln2 - hi rounded to fp32;
 *   Taylor coefficients 1/n! rounded to fp32;
 *   log series coefficients 2/(2j+1) rounded to fp32. */
static float c_log2e, c_ln2_hi, c_ln2_lo;
static float c_inv_fact[8];
static float c_log_series[5];
static pthread_once_t c_once = PTHREAD_ONCE_INIT;

static void init_constants(void) {
    long double ln2 = 0.693147180559945309417232121458176568L;
    c_log2e = (float)(1.0L / ln2);
    long double hi = roundl(ln2 * 65536.0L) / 65536.0L;
    c_ln2_hi = (float)hi;                 /* exact: 16 significant bits */
    c_ln2_lo = (float)(ln2 - hi);
    long double fact = 1.0L;
    for (int n = 0; n < 8; n++) {
        if (n > 0) fact *= n;
        c_inv_fact[n] = (float)(1.0L / fact);
    }
    for (int j = 1; j <= 4; j++) c_log_series[j] = (float)(2.0L / (2 * j + 1));
}

static void ensure_constants(void) { pthread_once(&c_once, init_constants); }

static float pow2i(int k) { return f_from_bits((uint32_t)(k + 127) << 23); }  /* -126..127 */

/* EXP(x): x = k*ln2 + r with k = nearest integer to x*log2(e) (ties to
 * even), r by two fused steps with the split ln2; e^r by the degree-7
 * Taylor polynomial in Horner form with fma; then 2^k applied as two
 * exact-power-of-two multiplies so that subnormal results round once. */
OR_EXPORT float or_expf(float x) {
    ensure_constants();
    if (x != x) return x + x;
    if (x > 89.0f) return INFINITY;
    if (x < -104.0f) return 0.0f;
    float kf = rintf(x * c_log2e);
    int k = (int)kf;
    float r = fmaf(-kf, c_ln2_hi, x);
    r = fmaf(-kf, c_ln2_lo, r);
    float p = c_inv_fact[7];
    p = fmaf(p, r, c_inv_fact[6]);
    p = fmaf(p, r, c_inv_fact[5]);
    p = fmaf(p, r, c_inv_fact[4]);
    p = fmaf(p, r, c_inv_fact[3]);
    p = fmaf(p, r, c_inv_fact[2]);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    int k1 = k >> 1;            /* floor(k/2) */
    int k2 = k - k1;
    return (p * pow2i(k1)) * pow2i(k2);
}

/* LOG(x): x = 2^k * m with m in [sqrt(1/2), sqrt(2)), f = m - 1 (exact),
 * s = f/(2+f), and log(1+f) = 2 atanh(s) = f - s*(f - R(s^2)) with
 * R(z) = sum_j 2 z^j/(2j+1), j = 1..4.  Written as
 * f - hfsq + s*(hfsq + R), hfsq = f*f/2, and recombined with k*ln2 split. */
OR_EXPORT float or_logf(float x) {
    ensure_constants();
    if (x != x) return x + x;
    if (x < 0.0f) return NAN;
    if (x == 0.0f) return -INFINITY;
    if (x == INFINITY) return x;
    uint32_t ix = bits_from_f(x);
    int k = 0;
    if (ix < 0x00800000u) {                 /* subnormal: scale by 2^25 */
        x = x * 33554432.0f;
        ix = bits_from_f(x);
        k = -25;
    }
    k += (int)(ix >> 23) - 127;
    uint32_t mant = ix & 0x007fffffu;
    float m;
    /* 0x3504f3 is the mantissa field of fp32(sqrt(2)) = 1.41421354 */
    if (mant > 0x3504f3u) { m = f_from_bits(mant | 0x3f000000u); k += 1; }
    else                  { m = f_from_bits(mant | 0x3f800000u); }
    float f = m - 1.0f;
    float s = f / (2.0f + f);
    float z = s * s;
    float R = fmaf(z, c_log_series[4], c_log_series[3]);
    R = fmaf(z, R, c_log_series[2]);
    R = fmaf(z, R, c_log_series[1]);
    R = z * R;
    float hfsq = (0.5f * f) * f;
    float kf = (float)k;
    return kf * c_ln2_hi - ((hfsq - (s * (hfsq + R) + kf * c_ln2_lo)) - f);
}

OR_EXPORT void or_expf_array(const float *x, float *y, int64_t n) {
    for (int64_t i = 0; i < n; i++) y[i] = or_expf(x[i]);
}
OR_EXPORT void or_logf_array(const float *x, float *y, int64_t n) {
    for (int64_t i = 0; i < n; i++) y[i] = or_logf(x[i]);
}
OR_EXPORT void or_f32_to_bf16_array(const float *x, uint16_t *y, int64_t n) {
    for (int64_t i = 0; i < n; i++) y[i] = or_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* GEMM (R1, R3).  C[i,j] = TREE over K/64 leaves; leaf b is the sum of      */
/* A[i,k]*W[j,k] for k in [64b, 64b+64) accumulated from +0 in K order.      */
/* A is [M,K] row-major (lda), W is [N,K] row-major (ldw).                   */
/* [ISO] 叁: fixed accumulation blocking.  [TBIK] Abstract: TP-invariant     */
/* matrix multiplication.  bf16*bf16 products have at most 16 significant    */
/* bits, so each product is exact in fp32 and fmaf equals mul-then-add.      */
/* ------------------------------------------------------------------------ */

#define LEAF 64

static void leaves_ij(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw,
                      int i, int j, int K, float *leaf) {
    int nb = K / LEAF;
    const uint16_t *a = A + (int64_t)i * lda;
    const uint16_t *w = W + (int64_t)j * ldw;
    for (int b = 0; b < nb; b++) {
        float c = 0.0f;
        for (int k = b * LEAF; k < (b + 1) * LEAF; k++)
            c = fmaf(or_bf16_to_f32(a[k]), or_bf16_to_f32(w[k]), c);
        leaf[b] = c;
    }
}

typedef struct {
    const uint16_t *A, *W;
    int64_t lda, ldw, ldc;
    float *C;
    int M, N, K, tp;
    float *ws;              /* tpsim partials [tp][M][N] or NULL */
    int nthreads, tid;
    /* sampled mode */
    const int32_t *rows, *cols;
    int64_t count;
    double *C64;            /* f64 mode */
    int mode;               /* 0 tree, 1 tpsim, 2 f64, 3 naive tp, 4 sampled */
} gemm_job;

static void *gemm_worker(void *p) {
    gemm_job *j = (gemm_job *)p;
    int nb = j->K / LEAF;
    float *leaf = (float *)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
    float *scratch = (float *)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
    int64_t total = (j->mode == 4) ? j->count : (int64_t)j->M * j->N;
    for (int64_t e = j->tid; e < total; e += j->nthreads) {
        int i, c;
        if (j->mode == 4) { i = j->rows[e]; c = j->cols[e]; }
        else { i = (int)(e / j->N); c = (int)(e % j->N); }
        if (j->mode == 2) {
            /* exact products, sequential double sum */
            const uint16_t *a = j->A + (int64_t)i * j->lda;
            const uint16_t *w = j->W + (int64_t)c * j->ldw;
            double s = 0.0;
            for (int k = 0; k < j->K; k++)
                s += (double)or_bf16_to_f32(a[k]) * (double)or_bf16_to_f32(w[k]);
            j->C64[(int64_t)i * j->ldc + c] = s;
            continue;
        }
        if (j->mode == 3) {
            /* negative control: each shard sums its K range sequentially,
             * shards are then added left to right */
            const uint16_t *a = j->A + (int64_t)i * j->lda;
            const uint16_t *w = j->W + (int64_t)c * j->ldw;
            int ks = j->K / j->tp;
            float total_s = 0.0f;
            for (int t = 0; t < j->tp; t++) {
                float part = 0.0f;
                for (int k = t * ks; k < (t + 1) * ks; k++)
                    part = fmaf(or_bf16_to_f32(a[k]), or_bf16_to_f32(w[k]), part);
                total_s = (t == 0) ? part : total_s + part;
            }
            j->C[(int64_t)i * j->ldc + c] = total_s;
            continue;
        }
        leaves_ij(j->A, j->lda, j->W, j->ldw, i, c, j->K, leaf);
        if (j->mode == 1) {
            float nodes[8];
            float r = or_tree_sharded(leaf, nb, j->tp, scratch, nodes);
            for (int t = 0; t < j->tp; t++)
                j->ws[((int64_t)t * j->M + i) * j->N + c] = nodes[t];
            j->C[(int64_t)i * j->ldc + c] = r;
        } else if (j->mode == 4) {
            j->C[e] = or_tree(leaf, nb, scratch);
        } else {
            j->C[(int64_t)i * j->ldc + c] = or_tree(leaf, nb, scratch);
        }
    }
    free(leaf);
    free(scratch);
    return NULL;
}

static void run_gemm(gemm_job *proto) {
    int nt = proto->nthreads < 1 ? 1 : proto->nthreads;
    if (nt > 256) nt = 256;
    pthread_t th[256];
    gemm_job jobs[256];
    for (int t = 0; t < nt; t++) {
        jobs[t] = *proto;
        jobs[t].nthreads = nt;
        jobs[t].tid = t;
    }
    for (int t = 1; t < nt; t++) pthread_create(&th[t], NULL, gemm_worker, &jobs[t]);
    gemm_worker(&jobs[0]);
    for (int t = 1; t < nt; t++) pthread_join(th[t], NULL);
}

/* Returns 0 on success, -2 when K is not a positive multiple of 64,
 * -3 when tp does not divide T. */
OR_EXPORT int or_gemm(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw,
                      float *C, int64_t ldc, int M, int N, int K, int nthreads) {
    if (K <= 0 || K % LEAF) return -2;
    gemm_job j = {0};
    j.A = A; j.W = W; j.lda = lda; j.ldw = ldw; j.ldc = ldc; j.C = C;
    j.M = M; j.N = N; j.K = K; j.nthreads = nthreads; j.mode = 0;
    run_gemm(&j);
    return 0;
}

/* Simulated tensor parallelism over K ([DT] 2.1.1: a row-parallel layer's  */
/* shards each produce a partial output and the partials are summed).        */
/* ws receives the tp shard nodes [tp][M][N]; C the combined result.         */
OR_EXPORT int or_gemm_tpsim(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw,
                            float *C, int64_t ldc, int M, int N, int K, int tp, float *ws,
                            int nthreads) {
    if (K <= 0 || K % LEAF) return -2;
    int T = or_tree_T(K / LEAF);
    if (tp < 1 || tp > T || T % tp) return -3;
    gemm_job j = {0};
    j.A = A; j.W = W; j.lda = lda; j.ldw = ldw; j.ldc = ldc; j.C = C;
    j.M = M; j.N = N; j.K = K; j.tp = tp; j.ws = ws; j.nthreads = nthreads; j.mode = 1;
    run_gemm(&j);
    return 0;
}

OR_EXPORT int or_gemm_f64(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw,
                          double *C, int64_t ldc, int M, int N, int K, int nthreads) {
    gemm_job j = {0};
    j.A = A; j.W = W; j.lda = lda; j.ldw = ldw; j.ldc = ldc; j.C64 = C;
    j.M = M; j.N = N; j.K = K; j.nthreads = nthreads; j.mode = 2;
    run_gemm(&j);
    return 0;
}

OR_EXPORT int or_gemm_naive_tp(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw,
                               float *C, int64_t ldc, int M, int N, int K, int tp,
                               int nthreads) {
    if (tp < 1 || K % tp) return -3;
    gemm_job j = {0};
    j.A = A; j.W = W; j.lda = lda; j.ldw = ldw; j.ldc = ldc; j.C = C;
    j.M = M; j.N = N; j.K = K; j.tp = tp; j.nthreads = nthreads; j.mode = 3;
    run_gemm(&j);
    return 0;
}

/* Selected outputs (rows[e], cols[e]) -> out[e]; for checks at full size. */
OR_EXPORT int or_gemm_sampled(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw,
                              int K, const int32_t *rows, const int32_t *cols, int64_t count,
                              float *out, int nthreads) {
    if (K <= 0 || K % LEAF) return -2;
    gemm_job j = {0};
    j.A = A; j.W = W; j.lda = lda; j.ldw = ldw; j.C = out; j.K = K;
    j.rows = rows; j.cols = cols; j.count = count; j.nthreads = nthreads; j.mode = 4;
    run_gemm(&j);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Rounding locations.  [ROUND] "the problem" and "three nodes": the aligned */
/* node keeps its intermediates in fp32 and rounds once, at its bf16 output; */
/* the misaligned stack rounds intermediates to bf16 along the way.  The     */
/* page does not list which intermediates; the reading taken here (R11) is   */
/* eager bf16 tensor arithmetic: every elementwise operation on bf16 operands */
/* is computed in fp32 and rounded to bf16, and fp32 tables are stored as    */
/* bf16.  `each_op` = 0: round once; 1: round after every operation.         */
/* ------------------------------------------------------------------------ */
static float bf_round(float v) { return or_bf16_to_f32(or_f32_to_bf16(v)); }

/* ------------------------------------------------------------------------ */
/* Residual-add + RMSNorm.  [ROUND] "three nodes": residual RMSNorm keeps    */
/* fp32 intermediates and rounds to bf16 once at the output.                 */
/*   h = x + r (fp32); r_out = bf16(h); ss = TREE(h*h); mean = ss/H;         */
/*   rstd = 1/sqrt(mean + eps); y = bf16((h*rstd)*w).                        */
/* each_op: h = bf16(x + r) before the norm, n = bf16(h*rstd), y = bf16(n*w). */
/* ------------------------------------------------------------------------ */
OR_EXPORT void or_rmsnorm_residual(const uint16_t *x, const uint16_t *r, const uint16_t *w,
                                   uint16_t *y, uint16_t *r_out, int rows, int H, int64_t ld,
                                   float eps, int each_op) {
    float *h = (float *)malloc(sizeof(float) * (size_t)H);
    float *sq = (float *)malloc(sizeof(float) * (size_t)H);
    float *scratch = (float *)malloc(sizeof(float) * (size_t)H);
    for (int i = 0; i < rows; i++) {
        const uint16_t *xi = x + (int64_t)i * ld;
        const uint16_t *ri = r + (int64_t)i * ld;
        for (int j = 0; j < H; j++) {
            h[j] = or_bf16_to_f32(xi[j]) + or_bf16_to_f32(ri[j]);
            if (each_op) h[j] = bf_round(h[j]);
            sq[j] = h[j] * h[j];
            r_out[(int64_t)i * ld + j] = or_f32_to_bf16(h[j]);
        }
        float ss = or_tree(sq, H, scratch);
        float mean = ss / (float)H;
        float rstd = 1.0f / sqrtf(mean + eps);
        for (int j = 0; j < H; j++) {
            float n = h[j] * rstd;
            if (each_op) n = bf_round(n);
            y[(int64_t)i * ld + j] = or_f32_to_bf16(n * or_bf16_to_f32(w[j]));
        }
    }
    free(h); free(sq); free(scratch);
}

/* ------------------------------------------------------------------------ */
/* RoPE.  [ROUND] "three nodes": the position-encoding node keeps fp32       */
/* intermediates.  Rotate-half pairing (i, i+d/2); each product rounded to   */
/* fp32 on its own, one bf16 rounding at the output.  each_op: the table    */
/* entries are rounded to bf16 and so is every product, then the difference */
/* and the sum are rounded (rotate_half arithmetic on bf16 tensors).         */
/* Table: angle(p,i) = p * theta^(-2i/d) in binary64, cos/sin in binary64,   */
/* one rounding to fp32.                                                     */
/* ------------------------------------------------------------------------ */
OR_EXPORT void or_rope_table(double theta, int head_dim, int max_pos, float *cos_tab,
                             float *sin_tab) {
    int half = head_dim / 2;
    for (int p = 0; p < max_pos; p++)
        for (int i = 0; i < half; i++) {
            double inv_freq = pow(theta, -(2.0 * i) / (double)head_dim);
            double ang = (double)p * inv_freq;
            cos_tab[(int64_t)p * half + i] = (float)cos(ang);
            sin_tab[(int64_t)p * half + i] = (float)sin(ang);
        }
}

OR_EXPORT void or_rope(const uint16_t *x, uint16_t *y, const int32_t *pos, const float *cos_tab,
                       const float *sin_tab, int T, int heads, int head_dim, int64_t ld_token,
                       int each_op) {
    int half = head_dim / 2;
    for (int t = 0; t < T; t++) {
        int p = pos[t];
        for (int hd = 0; hd < heads; hd++) {
            const uint16_t *xv = x + (int64_t)t * ld_token + (int64_t)hd * head_dim;
            uint16_t *yv = y + (int64_t)t * ld_token + (int64_t)hd * head_dim;
            for (int i = 0; i < half; i++) {
                float c = cos_tab[(int64_t)p * half + i];
                float s = sin_tab[(int64_t)p * half + i];
                float a = or_bf16_to_f32(xv[i]);
                float b = or_bf16_to_f32(xv[i + half]);
                float ac, bs, bc, as;
                if (each_op) {
                    c = bf_round(c); s = bf_round(s);
                    ac = bf_round(a * c); bs = bf_round(b * s);
                    bc = bf_round(b * c); as = bf_round(a * s);
                } else {
                    ac = a * c; bs = b * s; bc = b * c; as = a * s;
                }
                yv[i] = or_f32_to_bf16(ac - bs);
                yv[i + half] = or_f32_to_bf16(bc + as);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* SwiGLU.  [ROUND] "three nodes": the gated activation keeps fp32          */
/* intermediates.  y = bf16((g / (1 + EXP(-g))) * u).                        */
/* each_op: the activation is rounded first, y = bf16(bf16(silu(g)) * u).    */
/* ------------------------------------------------------------------------ */
OR_EXPORT void or_swiglu(const uint16_t *gate, const uint16_t *up, uint16_t *out, int rows,
                         int cols, int64_t ld_gate, int64_t ld_up, int64_t ld_out, int each_op) {
    for (int i = 0; i < rows; i++)
        for (int j = 0; j < cols; j++) {
            float g = or_bf16_to_f32(gate[(int64_t)i * ld_gate + j]);
            float u = or_bf16_to_f32(up[(int64_t)i * ld_up + j]);
            float den = 1.0f + or_expf(-g);
            float silu = g / den;
            if (each_op) silu = bf_round(silu);
            out[(int64_t)i * ld_out + j] = or_f32_to_bf16(silu * u);
        }
}

/* ------------------------------------------------------------------------ */
/* Training side: backward passes of the three nodes.  [TBIK] Abstract: the */
/* trainer (FSDP, TP = 1) and the inference engine must agree bit for bit;  */
/* [ROUND] "three nodes": the nodes keep fp32 intermediates and round once. */
/* The pages give no backward formulas; R12 takes the derivatives of the    */
/* forward definitions above, evaluated in fp32 in the order written here,  */
/* each output rounded once to bf16, and sums over tokens with TREE over    */
/* 64-token leaves (R1, R3) so that data-parallel shards are subtrees.      */
/* ------------------------------------------------------------------------ */

/* RoPE backward: the adjoint of the rotation is the rotation by -angle,
 *   dx[i] = bf16(dy[i]*c + dy[i+d/2]*s),  dx[i+d/2] = bf16(dy[i+d/2]*c - dy[i]*s),
 * each product rounded to fp32 separately. */
OR_EXPORT void or_rope_backward(const uint16_t *dy, uint16_t *dx, const int32_t *pos,
                                const float *cos_tab, const float *sin_tab, int T, int heads,
                                int head_dim, int64_t ld_token) {
    int half = head_dim / 2;
    for (int t = 0; t < T; t++) {
        int p = pos[t];
        for (int hd = 0; hd < heads; hd++) {
            const uint16_t *gv = dy + (int64_t)t * ld_token + (int64_t)hd * head_dim;
            uint16_t *ov = dx + (int64_t)t * ld_token + (int64_t)hd * head_dim;
            for (int i = 0; i < half; i++) {
                float c = cos_tab[(int64_t)p * half + i];
                float s = sin_tab[(int64_t)p * half + i];
                float a = or_bf16_to_f32(gv[i]);
                float b = or_bf16_to_f32(gv[i + half]);
                float ac = a * c, bs = b * s, bc = b * c, as = a * s;
                ov[i] = or_f32_to_bf16(ac + bs);
                ov[i + half] = or_f32_to_bf16(bc - as);
            }
        }
    }
}

/* SwiGLU backward for out = silu(g) * u, silu(g) = g * sigma(g):
 *   den = 1 + EXP(-g);  sig = 1 / den;  silu = g / den;
 *   du = bf16(dout * silu);
 *   dsilu = sig * (1 + g * (1 - sig));   dg = bf16((dout * u) * dsilu). */
OR_EXPORT void or_swiglu_backward(const uint16_t *gate, const uint16_t *up, const uint16_t *dout,
                                  uint16_t *dgate, uint16_t *dup, int rows, int cols,
                                  int64_t ld) {
    for (int i = 0; i < rows; i++)
        for (int j = 0; j < cols; j++) {
            int64_t o = (int64_t)i * ld + j;
            float g = or_bf16_to_f32(gate[o]);
            float u = or_bf16_to_f32(up[o]);
            float d = or_bf16_to_f32(dout[o]);
            float den = 1.0f + or_expf(-g);
            float sig = 1.0f / den;
            float silu = g / den;
            dup[o] = or_f32_to_bf16(d * silu);
            float dsilu = sig * (1.0f + g * (1.0f - sig));
            dgate[o] = or_f32_to_bf16((d * u) * dsilu);
        }
}

/* Residual RMSNorm backward.  Forward (above): h = x + r, rstd from TREE of
 * h*h, y = bf16((h*rstd)*w), r_out = bf16(h).  Given dy and the gradient
 * dr of the residual output (may be NULL = zero), per row:
 *   rstd as in the forward (same operations, same bits);
 *   g_j = dy_j * w_j;  dot = TREE_j(g_j * h_j);  c = (dot * ((rstd*rstd)*rstd)) / H;
 *   dh_j = bf16(((rstd * g_j) - (c * h_j)) + dr_j)      (dx = dr_in = dh);
 * and over the rows (tokens), for the weight:
 *   p_ij = dy_ij * (h_ij * rstd_i);  leaf b of column j = p_{64b,j} + ... +
 *   p_{64b+63,j} added in row order from +0;  dw_j = TREE over the leaves,
 *   evaluated as dp data-parallel shards (dp divides T) whose shard nodes
 *   are written to dw_shards [dp][H] when it is not NULL.
 * rows must be a multiple of 64 when dw is requested.  Returns 0 or -2/-3. */
OR_EXPORT int or_rmsnorm_backward(const uint16_t *x, const uint16_t *r, const uint16_t *w,
                                  const uint16_t *dy, const uint16_t *dr, uint16_t *dh,
                                  float *dw, int rows, int H, int64_t ld, float eps, int dp,
                                  float *dw_shards) {
    if (dw && (rows % LEAF)) return -2;
    int64_t nleaf = rows / LEAF;
    if (dw && nleaf > 0 && (dp < 1 || or_tree_T(nleaf) % dp)) return -3;
    float *h = (float *)malloc(sizeof(float) * (size_t)H);
    float *q = (float *)malloc(sizeof(float) * (size_t)H);
    float *scratch = (float *)malloc(sizeof(float) * (size_t)(H > nleaf ? H : nleaf));
    float *leaves = dw ? (float *)calloc((size_t)(nleaf > 0 ? nleaf : 1) * (size_t)H,
                                         sizeof(float)) : NULL;
    for (int i = 0; i < rows; i++) {
        const int64_t o = (int64_t)i * ld;
        for (int j = 0; j < H; j++) {
            h[j] = or_bf16_to_f32(x[o + j]) + or_bf16_to_f32(r[o + j]);
            q[j] = h[j] * h[j];
        }
        float ss = or_tree(q, H, scratch);
        float mean = ss / (float)H;
        float rstd = 1.0f / sqrtf(mean + eps);
        for (int j = 0; j < H; j++) {
            float g = or_bf16_to_f32(dy[o + j]) * or_bf16_to_f32(w[j]);
            q[j] = g * h[j];
        }
        float dot = or_tree(q, H, scratch);
        float c = (dot * ((rstd * rstd) * rstd)) / (float)H;
        for (int j = 0; j < H; j++) {
            float g = or_bf16_to_f32(dy[o + j]) * or_bf16_to_f32(w[j]);
            float v = (rstd * g) - (c * h[j]);
            if (dr) v = v + or_bf16_to_f32(dr[o + j]);
            dh[o + j] = or_f32_to_bf16(v);
            if (leaves) {
                float pr = or_bf16_to_f32(dy[o + j]) * (h[j] * rstd);
                float *lf = leaves + (int64_t)(i / LEAF) * H + j;
                *lf = *lf + pr;
            }
        }
    }
    if (dw) {
        float *col = (float *)malloc(sizeof(float) * (size_t)(nleaf > 0 ? nleaf : 1));
        for (int j = 0; j < H; j++) {
            for (int64_t b = 0; b < nleaf; b++) col[b] = leaves[b * H + j];
            float nodes[8];
            dw[j] = or_tree_sharded(col, nleaf, dp, scratch, nodes);
            if (dw_shards)
                for (int t = 0; t < dp; t++) dw_shards[(int64_t)t * H + j] = nleaf ? nodes[t] : 0.0f;
        }
        free(col);
    }
    free(h); free(q); free(scratch); free(leaves);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Log-softmax + target gather (R5).  [TBIK] Abstract: TP-invariant          */
/* reduction primitives; [ISO] 叁: train and inference logprobs compared     */
/* bit by bit.  Per row: m = max x; e_j = EXP(x_j - m); s = TREE(e) over V   */
/* (vocab shards = tree subtrees); lp = (x_t - m) - LOG(s).                  */
/* shard_nodes (optional) receives [M][tp] shard sums.                       */
/* ------------------------------------------------------------------------ */
OR_EXPORT int or_logsoftmax_gather(const float *logits, int64_t ld, const int32_t *targets,
                                   float *out, int M, int V, int tp, float *shard_nodes) {
    int T = or_tree_T(V);
    if (tp < 1 || tp > T || T % tp) return -3;
    float *e = (float *)malloc(sizeof(float) * (size_t)V);
    float *scratch = (float *)malloc(sizeof(float) * (size_t)V);
    for (int i = 0; i < M; i++) {
        const float *xr = logits + (int64_t)i * ld;
        float m = xr[0];
        for (int j = 1; j < V; j++) if (xr[j] > m) m = xr[j];
        for (int j = 0; j < V; j++) e[j] = or_expf(xr[j] - m);
        float nodes[8];
        float s = or_tree_sharded(e, V, tp, scratch, nodes);
        if (shard_nodes)
            for (int t = 0; t < tp; t++) shard_nodes[(int64_t)i * tp + t] = nodes[t];
        out[i] = (xr[targets[i]] - m) - or_logf(s);
    }
    free(e); free(scratch);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Causal softmax over attention scores (decoder composition).              */
/* S is fp32 [Lq, Lk] (ld_s); query row i sees keys j <= i + offset.        */
/* z_j = S[i,j]*scale; m = max over visible z; e_j = EXP(z_j - m) for        */
/* visible keys and +0 for masked ones; s = TREE(e) over all Lk entries;     */
/* P[i,j] = bf16(e_j / s).                                                   */
/* ------------------------------------------------------------------------ */
OR_EXPORT void or_softmax_causal(const float *S, int64_t ld_s, uint16_t *P, int64_t ld_p,
                                 int Lq, int Lk, int offset, float scale) {
    float *e = (float *)malloc(sizeof(float) * (size_t)Lk);
    float *z = (float *)malloc(sizeof(float) * (size_t)Lk);
    float *scratch = (float *)malloc(sizeof(float) * (size_t)Lk);
    for (int i = 0; i < Lq; i++) {
        int last = i + offset;        /* last visible key */
        float m = -INFINITY;
        for (int j = 0; j < Lk; j++) {
            z[j] = S[(int64_t)i * ld_s + j] * scale;
            if (j <= last && z[j] > m) m = z[j];
        }
        for (int j = 0; j < Lk; j++) e[j] = (j <= last) ? or_expf(z[j] - m) : 0.0f;
        float s = or_tree(e, Lk, scratch);
        for (int j = 0; j < Lk; j++) P[(int64_t)i * ld_p + j] = or_f32_to_bf16(e[j] / s);
    }
    free(e); free(z); free(scratch);
}
