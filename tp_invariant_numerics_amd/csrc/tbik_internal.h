// tbik_internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tbik {

// One GEMM launch: C[bat][part] = tree node over the groups of `part`.
struct GemmCall {
  const uint16_t *A; int64_t lda; int64_t strideA;
  const uint16_t *W; int64_t ldw; int64_t strideW;
  float *C; uint16_t *Cb; int64_t ldc; int64_t strideC;
  int64_t part_stride;   // element offset between the outputs of two parts
  int M, N, K, batch;
  int parts;             // K split into `parts` tree nodes (1 = the root)
  int leaf_mode;         // 0 MFMA, 1 scalar
  // When shard_of > 0 the K columns given are one shard of a tree over
  // tree_leaves leaves split into shard_of shards: the launch computes that
  // shard's node (its T/shard_of groups) and parts must be 1.
  int tree_leaves;
  int shard_of;
  // Optional: exact row maxima of C over 64-column blocks (needs C, one
  // batch, one part): pmax[row * ld_pmax + col / 64].
  float *pmax; int64_t ld_pmax;
  // Optional: SwiGLU epilogue instead of C (glu = 1 once, 2 each_op; W's
  // rows are [gate; up], N = 2F, H [M][F] bf16).  Ring kernel shapes only.
  uint16_t *H; int64_t ldh; int glu;
};

// Returns 0 or a TBIK_ERR_* code.
int launch_gemm(const GemmCall &c, hipStream_t s);
int gemm_split_parts(int M, int N, int K, int batch, int leaf_mode);
int launch_tree_combine(const float *ws, int tp, float *C, int64_t ldc, uint16_t *Cb, int M,
                        int N, hipStream_t s);
int launch_rmsnorm_residual(const uint16_t *x, const uint16_t *r, const uint16_t *w,
                            uint16_t *y, uint16_t *r_out, int rows, int H, int64_t ld,
                            float eps, int rounding, hipStream_t s);
int launch_rope(const uint16_t *x, uint16_t *y, const int32_t *pos, const float *cos_tab,
                const float *sin_tab, int T, int heads, int head_dim, int64_t ld_token,
                int max_pos, int rounding, hipStream_t s);
int launch_swiglu(const uint16_t *g, const uint16_t *u, uint16_t *o, int rows, int cols,
                  int64_t ldg, int64_t ldu, int64_t ldo, int rounding, hipStream_t s);
// launch_rope's rounding argument selecting the inverse rotation (backward)
constexpr int kRopeInverse = 100;
int launch_rope_backward(const uint16_t *dy, uint16_t *dx, const int32_t *pos,
                         const float *cos_tab, const float *sin_tab, int T, int heads,
                         int head_dim, int64_t ld_token, int max_pos, hipStream_t s);
int launch_swiglu_backward(const uint16_t *g, const uint16_t *u, const uint16_t *d, uint16_t *dg,
                           uint16_t *du, int rows, int cols, int64_t ldg, int64_t ldu,
                           int64_t ldd, int64_t lddg, int64_t lddu, hipStream_t s);
// Workspace of the RMSNorm backward, in floats: rstd per row (rounded up to
// 64 floats), then with dw the nleaf x H leaves and the dp x H shard nodes.
inline int64_t rmsnorm_bwd_rstd_floats(int rows) { return ((int64_t)rows + 63) / 64 * 64; }
inline int64_t rmsnorm_bwd_ws_floats(int rows, int H, int dp, bool want_dw) {
  int64_t n = rmsnorm_bwd_rstd_floats(rows);
  if (want_dw) n += (int64_t)(rows / 64) * H + (int64_t)dp * H;
  return n;
}
int launch_rmsnorm_backward(const uint16_t *x, const uint16_t *r, const uint16_t *w,
                            const uint16_t *dy, const uint16_t *dr, uint16_t *dh, float *dw,
                            int rows, int H, int64_t ld, float eps, int dp, float *ws,
                            hipStream_t s);
int launch_transpose_bf16(const uint16_t *x, int64_t ldx, uint16_t *y, int64_t ldy, int rows,
                          int cols, hipStream_t s);
int launch_logsoftmax(const float *logits, int64_t ld, const int32_t *targets, float *out,
                      int M, int V, int tp, float *ws, const float *pmax, int64_t ld_pmax,
                      int npmax, hipStream_t s);
int launch_softmax_causal(const float *S, int64_t ld_s, int64_t stride_s, uint16_t *P,
                          int64_t ld_p, int64_t stride_p, int Lq, int Lk, int batch, int offset,
                          float scale, hipStream_t s);
int launch_primitive(int op, const float *x, float *y, int64_t n, hipStream_t s);
int launch_attn_causal(const uint16_t *Q, int64_t ldq, const uint16_t *K, int64_t ldk,
                       const uint16_t *Vt, int64_t ldvt, uint16_t *O, int64_t ldo, int L, int heads,
                       int batch, float scale, hipStream_t s);
int launch_gather_rows(const uint16_t *table, int64_t ld_table, int rows, const int32_t *idx,
                       int n, int cols, uint16_t *out, int64_t ld_out, hipStream_t s);

// Maximum leaves per tree group supported by the kernels.
constexpr int kMaxGroupLeaves = 512;

}  // namespace tbik
