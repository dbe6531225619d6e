/*
 * oracle_sanitize.c -- drives every exported function of the CPU oracle on
 * small and edge-case shapes, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (host code only).  Out-of-bounds accesses,
 * use-after-free, leaks, signed overflow or invalid shifts abort the run;
 * a few cheap invariants (tensor-parallel shard counts give identical bits,
 * the tree of integers is exact) are checked on the way.
 *
 * The oracle is compiled into the same executable (its functions are
 * declared here by hand; no header is shared with the GPU library).
 *
 * Output: "ok calls=<n>" on success; exit status 1 on a failed invariant.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float or_bf16_to_f32(uint16_t h);
uint16_t or_f32_to_bf16(float f);
int or_tree_T(int64_t n);
float or_pair(const float *v, int64_t m, float *scratch);
float or_tree(const float *v, int64_t n, float *scratch);
float or_tree_sharded(const float *v, int64_t n, int tp, float *scratch, float *nodes);
float or_expf(float x);
float or_logf(float x);
void or_expf_array(const float *x, float *y, int64_t n);
void or_logf_array(const float *x, float *y, int64_t n);
void or_f32_to_bf16_array(const float *x, uint16_t *y, int64_t n);
int or_gemm(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw, float *C, int64_t ldc,
            int M, int N, int K, int nthreads);
int or_gemm_tpsim(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw, float *C,
                  int64_t ldc, int M, int N, int K, int tp, float *ws, int nthreads);
int or_gemm_f64(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw, double *C,
                int64_t ldc, int M, int N, int K, int nthreads);
int or_gemm_naive_tp(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw, float *C,
                     int64_t ldc, int M, int N, int K, int tp, int nthreads);
int or_gemm_sampled(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t ldw, int K,
                    const int32_t *rows, const int32_t *cols, int64_t count, float *out,
                    int nthreads);
void or_rmsnorm_residual(const uint16_t *x, const uint16_t *r, const uint16_t *w, uint16_t *y,
                         uint16_t *r_out, int rows, int H, int64_t ld, float eps, int each_op);
void or_rope_table(double theta, int head_dim, int max_pos, float *cos_tab, float *sin_tab);
void or_rope(const uint16_t *x, uint16_t *y, const int32_t *pos, const float *cos_tab,
             const float *sin_tab, int T, int heads, int head_dim, int64_t ld_token, int each_op);
void or_swiglu(const uint16_t *gate, const uint16_t *up, uint16_t *out, int rows, int cols,
               int64_t ld_gate, int64_t ld_up, int64_t ld_out, int each_op);
void or_rope_backward(const uint16_t *dy, uint16_t *dx, const int32_t *pos, const float *cos_tab,
                      const float *sin_tab, int T, int heads, int head_dim, int64_t ld_token);
void or_swiglu_backward(const uint16_t *gate, const uint16_t *up, const uint16_t *dout,
                        uint16_t *dgate, uint16_t *dup, int rows, int cols, int64_t ld);
int or_rmsnorm_backward(const uint16_t *x, const uint16_t *r, const uint16_t *w,
                        const uint16_t *dy, const uint16_t *dr, uint16_t *dh, float *dw, int rows,
                        int H, int64_t ld, float eps, int dp, float *dw_shards);
int or_logsoftmax_gather(const float *logits, int64_t ld, const int32_t *targets, float *out,
                         int M, int V, int tp, float *shard_nodes);
void or_softmax_causal(const float *S, int64_t ld_s, uint16_t *P, int64_t ld_p, int Lq, int Lk,
                       int offset, float scale);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {            /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float unif(void) { return (float)((next_u64() >> 40) * (1.0 / 16777216.0)) * 2.0f - 1.0f; }

static uint16_t *bf16_buf(size_t n, float scale) {
    uint16_t *b = (uint16_t *)malloc(sizeof(uint16_t) * (n ? n : 1));
    for (size_t i = 0; i < n; i++) b[i] = or_f32_to_bf16(unif() * scale);
    return b;
}
static float *f32_buf(size_t n, float scale) {
    float *b = (float *)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; i++) b[i] = unif() * scale;
    return b;
}

static int calls = 0, failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) { fprintf(stderr, "invariant failed: %s (line %d)\n", #c, __LINE__); failures++; } \
    } while (0)

static void gemm_case(int M, int N, int K, int64_t pad) {
    int64_t lda = K + pad, ldw = K + 2 * pad, ldc = N + pad;
    uint16_t *A = bf16_buf((size_t)M * lda, 2.0f), *W = bf16_buf((size_t)N * ldw, 0.1f);
    float *C = f32_buf((size_t)M * ldc, 0.0f), *C2 = f32_buf((size_t)M * ldc, 0.0f);
    double *C64 = (double *)malloc(sizeof(double) * (size_t)M * ldc);
    CHECK(or_gemm(A, lda, W, ldw, C, ldc, M, N, K, 3) == 0); calls++;
    CHECK(or_gemm_f64(A, lda, W, ldw, C64, ldc, M, N, K, 2) == 0); calls++;
    int T = or_tree_T(K / 64);
    for (int tp = 1; tp <= T; tp *= 2) {
        float *ws = f32_buf((size_t)tp * M * N, 0.0f);
        CHECK(or_gemm_tpsim(A, lda, W, ldw, C2, ldc, M, N, K, tp, ws, 2) == 0); calls++;
        for (int i = 0; i < M; i++)
            CHECK(memcmp(C + (int64_t)i * ldc, C2 + (int64_t)i * ldc, sizeof(float) * N) == 0);
        free(ws);
    }
    CHECK(or_gemm_naive_tp(A, lda, W, ldw, C2, ldc, M, N, K, 1, 1) == 0); calls++;
    int64_t cnt = 5;
    int32_t rows[5], cols[5];
    float out[5];
    for (int e = 0; e < cnt; e++) { rows[e] = (int)(next_u64() % M); cols[e] = (int)(next_u64() % N); }
    CHECK(or_gemm_sampled(A, lda, W, ldw, K, rows, cols, cnt, out, 2) == 0); calls++;
    for (int e = 0; e < cnt; e++) CHECK(memcmp(&out[e], &C[(int64_t)rows[e] * ldc + cols[e]], 4) == 0);
    /* invalid shapes are rejected, not read */
    CHECK(or_gemm(A, lda, W, ldw, C, ldc, M, N, K + 1, 1) == -2); calls++;
    CHECK(or_gemm_tpsim(A, lda, W, ldw, C, ldc, M, N, K, 16, NULL, 1) == -3); calls++;
    free(A); free(W); free(C); free(C2); free(C64);
}

int main(void) {
    /* primitives */
    float xs[9] = {0.0f, -0.0f, 1.0f, -1.0f, 88.7f, -103.9f, INFINITY, -INFINITY, NAN};
    float ys[9];
    uint16_t hs[9];
    or_expf_array(xs, ys, 9); calls++;
    or_logf_array(xs, ys, 9); calls++;
    or_f32_to_bf16_array(xs, hs, 9); calls++;
    for (int i = 0; i < 9; i++) { (void)or_expf(xs[i]); (void)or_logf(xs[i]); (void)or_bf16_to_f32(hs[i]); }
    for (int64_t n = 1; n <= 300; n++) CHECK(or_tree_T(n) >= 1);

    /* trees: every n up to 600, integer data exact, shard counts agree */
    for (int64_t n = 1; n <= 600; n++) {
        float *v = f32_buf((size_t)n, 0.0f), *s = f32_buf((size_t)n, 0.0f);
        double exact = 0.0;
        for (int64_t i = 0; i < n; i++) { v[i] = (float)((int64_t)(next_u64() % 2001) - 1000); exact += v[i]; }
        float t = or_tree(v, n, s);
        CHECK((double)t == exact);
        (void)or_pair(v, n, s);
        int T = or_tree_T(n);
        for (int tp = 1; tp <= T; tp *= 2) {
            float nodes[8];
            float r = or_tree_sharded(v, n, tp, s, nodes);
            CHECK(memcmp(&r, &t, 4) == 0);
        }
        calls += 3;
        free(v); free(s);
    }

    /* GEMM: one leaf, ragged, 28-leaf and 11-leaf groups, strided */
    gemm_case(1, 1, 64, 0);
    gemm_case(3, 5, 64 * 3, 7);
    gemm_case(4, 3, 64 * 28, 0);
    gemm_case(2, 6, 64 * 88, 5);
    gemm_case(5, 2, 64 * 224, 0);

    /* row nodes */
    for (int H = 1; H <= 4104; H = H * 3 + 5) {
        int rows = 3;
        int64_t ld = H + 3;
        uint16_t *x = bf16_buf((size_t)rows * ld, 3.0f), *r = bf16_buf((size_t)rows * ld, 3.0f);
        uint16_t *w = bf16_buf((size_t)H, 1.0f), *y = bf16_buf((size_t)rows * ld, 0.0f);
        uint16_t *ro = bf16_buf((size_t)rows * ld, 0.0f), *dh = bf16_buf((size_t)rows * ld, 0.0f);
        for (int e = 0; e < 2; e++) { or_rmsnorm_residual(x, r, w, y, ro, rows, H, ld, 1e-6f, e); calls++; }
        float *dw = f32_buf((size_t)H, 0.0f), *sh = f32_buf((size_t)8 * H, 0.0f);
        /* weight gradients need whole 64-token leaves: 3 rows are rejected */
        CHECK(or_rmsnorm_backward(x, r, w, y, ro, dh, dw, rows, H, ld, 1e-6f, 1, sh) != 0); calls++;
        CHECK(or_rmsnorm_backward(x, r, w, y, NULL, dh, NULL, rows, H, ld, 1e-6f, 1, NULL) == 0); calls++;
        free(x); free(r); free(w); free(y); free(ro); free(dh); free(dw); free(sh);
    }
    {
        int rows = 128, H = 96;
        uint16_t *x = bf16_buf((size_t)rows * H, 3.0f), *r = bf16_buf((size_t)rows * H, 3.0f);
        uint16_t *w = bf16_buf((size_t)H, 1.0f), *dy = bf16_buf((size_t)rows * H, 1.0f);
        uint16_t *dr = bf16_buf((size_t)rows * H, 1.0f), *dh = bf16_buf((size_t)rows * H, 0.0f);
        float *dw = f32_buf((size_t)H, 0.0f), *sh = f32_buf((size_t)2 * H, 0.0f);
        CHECK(or_rmsnorm_backward(x, r, w, dy, dr, dh, dw, rows, H, H, 1e-6f, 2, sh) == 0); calls++;
        free(x); free(r); free(w); free(dy); free(dr); free(dh); free(dw); free(sh);
    }
    {
        int T = 9, heads = 3, hd = 16, maxp = 40;
        int64_t ld = heads * hd + 4;
        float *ct = f32_buf((size_t)maxp * hd / 2, 0.0f), *st = f32_buf((size_t)maxp * hd / 2, 0.0f);
        or_rope_table(1e6, hd, maxp, ct, st); calls++;
        int32_t pos[9];
        for (int t = 0; t < T; t++) pos[t] = (int32_t)(next_u64() % maxp);
        uint16_t *x = bf16_buf((size_t)T * ld, 2.0f), *y = bf16_buf((size_t)T * ld, 0.0f);
        for (int e = 0; e < 2; e++) { or_rope(x, y, pos, ct, st, T, heads, hd, ld, e); calls++; }
        or_rope_backward(x, y, pos, ct, st, T, heads, hd, ld); calls++;
        free(ct); free(st); free(x); free(y);
    }
    {
        int rows = 4, cols = 37;
        uint16_t *g = bf16_buf((size_t)rows * cols, 100.0f), *u = bf16_buf((size_t)rows * cols, 2.0f);
        uint16_t *o = bf16_buf((size_t)rows * cols, 0.0f), *o2 = bf16_buf((size_t)rows * cols, 0.0f);
        for (int e = 0; e < 2; e++) { or_swiglu(g, u, o, rows, cols, cols, cols, cols, e); calls++; }
        or_swiglu_backward(g, u, o, o, o2, rows, cols, cols); calls++;
        free(g); free(u); free(o); free(o2);
    }
    /* log-softmax: V from 1 to a few thousand, every valid tp */
    for (int V = 1; V <= 3000; V = V * 2 + 3) {
        int M = 3;
        int64_t ld = V + 1;
        float *lg = f32_buf((size_t)M * ld, 20.0f), *out = f32_buf((size_t)M, 0.0f);
        int32_t tg[3] = {0, V - 1, V / 2};
        float nodes1[3], lp1[3];
        CHECK(or_logsoftmax_gather(lg, ld, tg, lp1, M, V, 1, nodes1) == 0); calls++;
        int T = or_tree_T(V);
        for (int tp = 2; tp <= T; tp *= 2) {
            float nodes[3 * 8];
            CHECK(or_logsoftmax_gather(lg, ld, tg, out, M, V, tp, nodes) == 0); calls++;
            CHECK(memcmp(out, lp1, sizeof(lp1)) == 0);
        }
        float junk[3 * 16];
        CHECK(or_logsoftmax_gather(lg, ld, tg, out, M, V, 16, junk) == -3); calls++;
        free(lg); free(out);
    }
    /* causal softmax with an offset and ragged lengths */
    for (int Lk = 1; Lk <= 200; Lk += 37) {
        int Lq = Lk > 3 ? Lk - 3 : 1;
        float *S = f32_buf((size_t)Lq * Lk, 30.0f);
        uint16_t *P = bf16_buf((size_t)Lq * Lk, 0.0f);
        or_softmax_causal(S, Lk, P, Lk, Lq, Lk, Lk - Lq, 0.0883883476f); calls++;
        free(S); free(P);
    }
    if (failures) { fprintf(stderr, "%d invariants failed\n", failures); return 1; }
    printf("ok calls=%d\n", calls);
    return 0;
}
