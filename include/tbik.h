/*
 * tbik.h -- C ABI of libtbik.so: tree-based invariant kernels (TBIK) for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes comes from these web pages:
 *  [TBIK]  "Deterministic Inference across Tensor Parallel Sizes That
 *          Eliminates Training-Inference Mismatch" (Zhang et al.), summary
 *          page: Abstract (TP-invariant matmul and reduction primitives;
 *          intra- and inter-GPU reduction orders aligned by one hierarchical
 *          binary tree); "technical framework" (shard, reduce locally per
 *          GPU, then combine GPUs by a binary tree); "key design".
 *  [ROUND] winzheng.jp article on rounding-location alignment (Ke, Cai,
 *          Wang), "surgical fix: three nodes": RoPE, SwiGLU and residual
 *          RMSNorm keep fp32 intermediates and round to bf16 only at the
 *          output.
 *  [ISO]   nxmr.cn brief on SkyRL IsoExec, section 叁: an execution contract
 *          with a fixed accumulation blocking; train and inference logprobs
 *          compared bit by bit.
 *  [DT]    "09｜分布式训练、数值稳定性与评测证据", section 2.1.1: a row-
 *          parallel layer's shards each produce a full-shape partial output
 *          that is summed.
 *  [ND]    "01-推理阶段的非确定性", sections 2 and 5: the order of a
 *          parallel sum, and atomics, change results.
 *
 * THE TREE.  Every fp32 reduction in this library (GEMM over K, row sums)
 * follows one fixed tree over n leaves: T = the largest power of two <= 8
 * dividing n; group g holds leaves [g*n/T, (g+1)*n/T); inside a group,
 * neighbours are added level by level and an odd last element moves up one
 * level unchanged; the T group sums are combined by a perfect binary tree.
 * A tensor-parallel shard t of tp (tp | T) owns groups [t*T/tp,(t+1)*T/tp):
 * its partial is a node of the tree, and combining the tp partials is the
 * tree's top log2(tp) levels.  Results are therefore bit-identical for any
 * tp in {1,2,4,8} that divides T, for any batch size, and for any launch
 * configuration.  No kernel uses atomics.
 *
 * CONVENTIONS (all entry points).
 *  - bf16 values are passed as 16-bit patterns (tbik_bf16).
 *  - Every data pointer is DEVICE memory owned by the caller; the library
 *    never allocates, frees or keeps a pointer after the call returns.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  Outputs are valid once the stream reaches the call.
 *  - Arguments are validated on the host before any launch; an invalid
 *    call returns a negative TBIK_ERR_* code and launches nothing.
 *  - Pointers must be aligned to their element size.  GEMM operands A and
 *    W (and RoPE's tensors and tables) must also be 16-byte aligned with
 *    leading dimensions (in elements) that are multiples of 8; violations
 *    return TBIK_ERR_ALIGN.  Other arrays take any leading dimension >= the
 *    row length; wider memory accesses are used when alignment permits,
 *    which never changes a result bit nor the set of accepted shapes
 *    (size limits below depend on the shape only).
 *  - Outputs must not overlap inputs unless stated otherwise.
 *  - Inputs must be finite; non-finite inputs give unspecified values (but
 *    never out-of-bounds accesses).
 *  - Entry points are thread-safe (the only global state is the per-device
 *    address of tbik_gemm_noalloc's scratch array, set once under a lock).
 */
#ifndef TBIK_H
#define TBIK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t tbik_bf16;

enum {
    TBIK_OK = 0,
    TBIK_ERR_NULL = -1,       /* a required pointer is NULL                     */
    TBIK_ERR_SHAPE = -2,      /* a size is negative, K % 64 != 0, ld too small  */
    TBIK_ERR_TP = -3,         /* tp not in {1,2,4,8} or does not divide T       */
    TBIK_ERR_ALIGN = -4,      /* pointer not 16-byte aligned or ld % 8 != 0     */
    TBIK_ERR_WORKSPACE = -5,  /* workspace missing or too small                 */
    TBIK_ERR_LAUNCH = -6,     /* the HIP runtime rejected a launch              */
    TBIK_ERR_ARG = -7         /* another argument is out of range               */
};

enum { TBIK_LEAF_MFMA = 0, TBIK_LEAF_SCALAR = 1 };

/* Library version as major*10000 + minor*100 + patch. */
int tbik_version(void);

/* Static description of an error code (never NULL). */
const char *tbik_strerror(int code);

/* T of the tree over n leaves (1, 2, 4 or 8); 0 when n <= 0. */
int tbik_tree_groups(int64_t n);

/* ------------------------------------------------------------------------
 * GEMM:  C[i,j] = TREE_b( leaf_b(i,j) ),  b = 0 .. K/64-1,
 *        leaf_b(i,j) = sum_{k=64b}^{64b+63} A[i,k] * W[j,k]   (fp32, from +0)
 * [TBIK] Abstract (TP-invariant matrix multiplication); [ISO] 叁 (fixed
 * accumulation blocking: 64-wide K blocks).
 *
 *  A       [M, K] bf16, row-major, row stride lda (elements)
 *  W       [N, K] bf16, row-major, row stride ldw (the nn.Linear layout)
 *  C       [M, N] fp32, row stride ldc; may be NULL if C_bf16 is given
 *  C_bf16  [M, N] bf16 (round-to-nearest-even of C), row stride ldc; NULL
 *          to skip.  At least one of C, C_bf16 is required.
 *  K       positive multiple of 64.
 *  leaf_mode
 *    TBIK_LEAF_MFMA    a leaf is two chained v_mfma_f32_16x16x32_bf16 from a
 *                      zero accumulator (k 0..31 then 32..63 of the block).
 *                      The same instruction sequence is used for every
 *                      shape, tile and tp, so the bits do not depend on M,
 *                      on the row's position in the batch or on tp.
 *    TBIK_LEAF_SCALAR  a leaf is 64 sequential fp32 fma in increasing k;
 *                      bit-exact with the CPU oracle.  Slow; for checking.
 *  ws, ws_bytes
 *          optional device workspace (NULL / 0: none; 16-byte aligned).
 *          When it holds tbik_gemm_workspace_bytes(M, N, K) bytes and that
 *          is non-zero, K is split into 2, 4 or 8 aligned nodes of the tree
 *          computed by separate workgroups into ws and combined by the top
 *          of the tree (the same bits as without: the split is at tree
 *          nodes; TBIK summary page, "technical framework").  Worth it when
 *          M x N has too few tiles to occupy the GPU, and for M <= 32 at
 *          K = 14336, where each of the 8 parts reads only its own K slice
 *          of A.  The contents of ws are unspecified afterwards.
 * ---------------------------------------------------------------------- */
size_t tbik_gemm_workspace_bytes(int M, int N, int K);

int tbik_gemm(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw,
              float *C, int64_t ldc, tbik_bf16 *C_bf16, int M, int N, int K,
              int leaf_mode, float *ws, size_t ws_bytes, void *stream);

/* Strided-batched form: for b in [0,batch): A + b*strideA, W + b*strideW,
 * C + b*strideC, C_bf16 + b*strideC (strides in elements, multiples of 8).
 * Each batch entry is computed exactly as tbik_gemm would compute it. */
int tbik_gemm_strided_batched(const tbik_bf16 *A, int64_t lda, int64_t strideA,
                              const tbik_bf16 *W, int64_t ldw, int64_t strideW,
                              float *C, int64_t ldc, int64_t strideC, tbik_bf16 *C_bf16,
                              int M, int N, int K, int batch, int leaf_mode, void *stream);

/* ------------------------------------------------------------------------
 * Simulated tensor-parallel GEMM ([DT] 2.1.1 row-parallel partial sums;
 * [TBIK] "technical framework").  K is split into tp shards aligned with
 * the tree's groups; shard t computes its partial P_t (a node of the tree)
 * into ws[t] = ws + t*M*N (fp32, dense [M,N]); a combine kernel then runs
 * the top log2(tp) levels of the tree over the tp partials into C/C_bf16.
 * The result is bit-identical to tbik_gemm with the same leaf_mode.  ws
 * keeps the partials after the call (they are what real TP would exchange).
 *  tp      1, 2, 4 or 8; must divide T of the tree over K/64 leaves.
 *  ws      device workspace of at least tbik_gemm_tpsim_workspace_bytes().
 * ---------------------------------------------------------------------- */
size_t tbik_gemm_tpsim_workspace_bytes(int M, int N, int K, int tp);

int tbik_gemm_tpsim(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw,
                    float *C, int64_t ldc, tbik_bf16 *C_bf16, int M, int N, int K, int tp,
                    int leaf_mode, float *ws, size_t ws_bytes, void *stream);

/* Only the partial step of tbik_gemm_tpsim: all tp shard partials in one
 * launch, ws[t] = ws + t*M*N (dense [M,N] fp32).  Same validation as
 * tbik_gemm_tpsim (ws must hold tp*M*N floats). */
int tbik_gemm_tp_partials(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw,
                          float *ws, size_t ws_bytes, int M, int N, int K, int tp, int leaf_mode,
                          void *stream);

/* One rank's share of real tensor parallelism ([DT] 2.1.1; [TBIK]
 * "technical framework": reduce locally, then combine across GPUs).
 *  A_t  [M, K_total/tp] bf16: this rank's K slice of the activations
 *  W_t  [N, K_total/tp] bf16: this rank's K slice of the weight rows
 *  P    [M, N] fp32 (row stride ldp): this shard's node of the tree over
 *       the K_total/64 leaves -- bit-identical to ws[t] of tbik_gemm_tpsim
 *       for the shard whose columns are given.  tp | T of the full tree.
 * Combining the tp ranks' P (gathered into a dense [tp][M][N] buffer) with
 * tbik_tree_combine reproduces tbik_gemm bit for bit. */
int tbik_gemm_shard(const tbik_bf16 *A_t, int64_t lda, const tbik_bf16 *W_t, int64_t ldw,
                    float *P, int64_t ldp, int M, int N, int K_total, int tp, int leaf_mode,
                    void *stream);

/* Only the combine step of tbik_gemm_tpsim: C = top tree over ws[0..tp-1]
 * (dense [tp][M][N] fp32 partials).  Lets a caller that produced the
 * partials elsewhere (e.g. on several GPUs) finish the same tree. */
int tbik_tree_combine(const float *ws, int tp, float *C, int64_t ldc, tbik_bf16 *C_bf16,
                      int M, int N, void *stream);

/* ------------------------------------------------------------------------
 * Rounding location of the three nodes below ([ROUND] "the problem", "three
 * nodes"): the aligned node keeps every intermediate in fp32 and rounds once,
 * at its bf16 output (what tbik_rmsnorm_residual, tbik_rope and tbik_swiglu
 * compute); the misaligned stack the article describes rounds intermediates
 * to bf16 along the way.  TBIK_ROUND_EACH_OP is that stack read as eager
 * bf16 tensor arithmetic: every elementwise operation is computed in fp32
 * and rounded to bf16, and fp32 tables are stored as bf16.  The _ex entry
 * points take one of these; any other value returns TBIK_ERR_ARG.
 * ---------------------------------------------------------------------- */
enum { TBIK_ROUND_ONCE = 0, TBIK_ROUND_EACH_OP = 1 };

/* ------------------------------------------------------------------------
 * Fused residual-add + RMSNorm ([ROUND] "three nodes"; [TBIK] reduction
 * primitives).  Per row, all intermediates fp32:
 *   h = x + r;  r_out = bf16(h);  ss = TREE_j(h_j * h_j);  mean = ss / H;
 *   rstd = 1 / sqrt(mean + eps)   (correctly rounded divide and sqrt);
 *   y = bf16((h * rstd) * w).
 *  x, r, y, r_out  [rows, H] bf16 with row stride ld; r_out may be NULL.
 *  w               [H] bf16.
 *  H               1 .. 65536, any value, at any alignment of the rows
 *                  (groups whose size has few factors of two are reduced
 *                  over 16-leaf chunks plus a tail item, the same tree);
 *                  eps >= 0.
 * ---------------------------------------------------------------------- */
int tbik_rmsnorm_residual(const tbik_bf16 *x, const tbik_bf16 *r, const tbik_bf16 *w,
                          tbik_bf16 *y, tbik_bf16 *r_out, int rows, int H, int64_t ld,
                          float eps, void *stream);

/* tbik_rmsnorm_residual with a rounding location.  TBIK_ROUND_EACH_OP:
 *   h = bf16(x + r) (the residual output, and the input of the norm);
 *   ss, rstd as above from that h;  y = bf16(bf16(h * rstd) * w). */
int tbik_rmsnorm_residual_ex(const tbik_bf16 *x, const tbik_bf16 *r, const tbik_bf16 *w,
                             tbik_bf16 *y, tbik_bf16 *r_out, int rows, int H, int64_t ld,
                             float eps, int rounding, void *stream);

/* ------------------------------------------------------------------------
 * RoPE, rotate-half pairing ([ROUND] "three nodes": fp32 intermediates).
 * For token t, head h, i < d/2, with c = cos_tab[pos[t], i], s = sin_tab[..]:
 *   y[i]       = bf16(x[i]*c - x[i+d/2]*s)
 *   y[i+d/2]   = bf16(x[i+d/2]*c + x[i]*s)
 * each product rounded to fp32 separately (no fma).
 *  x, y      [T, heads, d] bf16; token stride ld_token >= heads*d; heads
 *            contiguous with stride d.  y == x (in place) is allowed.
 *  pos       [T] int32, each in [0, max_pos) (out-of-range positions are
 *            clamped to the table; the result is then unspecified).
 *  cos_tab, sin_tab  [max_pos, d/2] fp32 (see tbik_rope_table).
 *  d         even, 2 .. 1024, d/2 a multiple of 4.
 * ---------------------------------------------------------------------- */
int tbik_rope(const tbik_bf16 *x, tbik_bf16 *y, const int32_t *pos, const float *cos_tab,
              const float *sin_tab, int T, int heads, int head_dim, int64_t ld_token,
              int max_pos, void *stream);

/* tbik_rope with a rounding location.  TBIK_ROUND_EACH_OP: c = bf16(c),
 * s = bf16(s), every product rounded to bf16, then
 *   y[i] = bf16(bf16(x[i]*c) - bf16(x[i+d/2]*s)),
 *   y[i+d/2] = bf16(bf16(x[i+d/2]*c) + bf16(x[i]*s)). */
int tbik_rope_ex(const tbik_bf16 *x, tbik_bf16 *y, const int32_t *pos, const float *cos_tab,
                 const float *sin_tab, int T, int heads, int head_dim, int64_t ld_token,
                 int max_pos, int rounding, void *stream);

/* HOST helper: cos_tab/sin_tab (host memory, [max_pos, d/2] fp32) with
 * angle = p * theta^(-2i/d) evaluated in binary64 and cos/sin rounded once
 * to fp32 (an fp32 angle would lose ~1e-3 rad at p ~ 3e4). */
int tbik_rope_table(double theta, int head_dim, int max_pos, float *cos_tab, float *sin_tab);

/* ------------------------------------------------------------------------
 * SwiGLU ([ROUND] "three nodes"): out = bf16((g / (1 + EXP(-g))) * u), all
 * fp32, one correctly rounded division.  EXP is the library's fp32
 * exponential (Cody-Waite reduction, degree-7 Taylor polynomial; < 1 ulp).
 *  gate, up, out  [rows, cols] bf16 with row strides ld_gate, ld_up, ld_out.
 * ---------------------------------------------------------------------- */
int tbik_swiglu(const tbik_bf16 *gate, const tbik_bf16 *up, tbik_bf16 *out, int rows,
                int cols, int64_t ld_gate, int64_t ld_up, int64_t ld_out, void *stream);

/* tbik_swiglu with a rounding location.  TBIK_ROUND_EACH_OP:
 *   out = bf16(bf16(g / (1 + EXP(-g))) * u). */
int tbik_swiglu_ex(const tbik_bf16 *gate, const tbik_bf16 *up, tbik_bf16 *out, int rows,
                   int cols, int64_t ld_gate, int64_t ld_up, int64_t ld_out, int rounding,
                   void *stream);

/* ------------------------------------------------------------------------
 * Gate/up projection with the SwiGLU node fused into its epilogue: for the
 * decoder's FFN ([TBIK] the invariant GEMM; [ROUND] "three nodes").
 *   G = A W_g^T, U = A W_u^T      the tree GEMM (MFMA leaves), W_gu = [W_g; W_u]
 *   H = SwiGLU(bf16(G), bf16(U))  as tbik_swiglu_ex with `rounding`
 * H holds exactly what tbik_gemm (bf16 output over W_gu) followed by
 * tbik_swiglu_ex on its two column halves returns, without writing G and U.
 *  A     [M, K] bf16, row stride lda;  W_gu [2F, K] bf16, row stride ldw
 *        (rows 0..F-1 the gate weights, F..2F-1 the up weights).
 *  H     [M, F] bf16, row stride ldh >= F (2-byte aligned).
 *  F     a positive multiple of 16.
 * Supported where the LDS-ring GEMM kernel runs the whole tree: M > 32, K's
 * groups of a size that kernel takes (K = 1024 .. 14336 in the decoder and
 * benchmark shapes), 2F * ldw * 2 bytes < 2^31; otherwise TBIK_ERR_SHAPE and
 * nothing is launched (compose tbik_gemm and tbik_swiglu_ex instead).
 * ---------------------------------------------------------------------- */
int tbik_gemm_swiglu(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W_gu, int64_t ldw,
                     tbik_bf16 *H, int64_t ldh, int M, int F, int K, int rounding, void *stream);

/* ------------------------------------------------------------------------
 * Log-softmax + target gather ([TBIK] reduction primitives; [ISO] 叁 logprob
 * comparison).  Per row i:
 *   m = max_j x_j (exact);  e_j = EXP(x_j - m);  s = TREE_j(e_j);
 *   out_lp[i] = (x_{t_i} - m) - LOG(s).
 * The tree's T groups are the vocab-parallel shards: with tp > 1 the
 * library materialises each shard's partial sum in ws (what vocab-parallel
 * ranks would exchange) and combines them with the top of the tree; the
 * result is bit-identical for every tp.
 *  logits   [M, V] fp32, row stride ld.  M <= 65535; a row's chunk sums
 *           are staged in LDS: T * ceil((V / T) / 16) <= 40944, i.e. any V
 *           up to about 655000 (655104 when V / T is a multiple of 16), at
 *           any alignment of the rows; larger V return TBIK_ERR_SHAPE
 *           before any launch.
 *  targets  [M] int32 in [0, V) (out-of-range targets: out_lp = NaN).
 *  out_lp   [M] fp32.
 *  ws       at least tbik_logsoftmax_workspace_bytes(M, V, tp) = M*tp*4
 *           bytes; on return ws[i*tp + t] holds row i's shard-t sum.
 * ---------------------------------------------------------------------- */
size_t tbik_logsoftmax_workspace_bytes(int M, int V, int tp);

int tbik_logsoftmax_gather(const float *logits, int64_t ld, const int32_t *targets,
                           float *out_lp, int M, int V, int tp, float *ws, size_t ws_bytes,
                           void *stream);

/* ------------------------------------------------------------------------
 * The logprob path with the row maximum fused into the LM-head GEMM
 * ([TBIK] Abstract; [ISO] 叁).  The maximum is exact in any order, so
 * per-block maxima taken in the GEMM's epilogue give the same m, and the
 * log-softmax then reads the logits from HBM once instead of twice.
 *
 * tbik_gemm_logits: C = tbik_gemm(A, W) with MFMA leaves (fp32 C required)
 * and pmax[i*ld_pmax + b] = max of C[i, 64b .. 64b+63] (clipped to N) for
 * b < ceil(N/64).  ld_pmax >= ceil(N/64); pmax 4-byte aligned.
 *
 * tbik_logsoftmax_gather_pmax: tbik_logsoftmax_gather with
 * m_i = max_b pmax[i*ld_pmax + b] over b < npmax instead of a pass over the
 * logits.  Defined only if that maximum equals the row maximum of the
 * logits (as tbik_gemm_logits guarantees with npmax = ceil(V/64)); the
 * result is then bit-identical to tbik_gemm + tbik_logsoftmax_gather.
 * ---------------------------------------------------------------------- */
int tbik_gemm_logits(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw,
                     float *C, int64_t ldc, int M, int N, int K, float *pmax, int64_t ld_pmax,
                     void *stream);

int tbik_logsoftmax_gather_pmax(const float *logits, int64_t ld, const int32_t *targets,
                                float *out_lp, int M, int V, int tp, const float *pmax,
                                int64_t ld_pmax, int npmax, float *ws, size_t ws_bytes,
                                void *stream);

/* ------------------------------------------------------------------------
 * Causal softmax over attention scores (decoder composition).
 *   z_j = S[i,j] * scale;  visible keys j <= i + offset;
 *   m = max of visible z;  e_j = EXP(z_j - m) if visible else +0;
 *   s = TREE_j(e_j) over all Lk keys;  P[i,j] = bf16(e_j / s).
 *  S  [batch][Lq, Lk] fp32 (row stride ld_s, batch stride stride_s)
 *  P  [batch][Lq, Lk] bf16 (row stride ld_p, batch stride stride_p)
 *  offset >= 0;  Lk <= 65536.
 * ---------------------------------------------------------------------- */
int tbik_softmax_causal(const float *S, int64_t ld_s, int64_t stride_s, tbik_bf16 *P,
                        int64_t ld_p, int64_t stride_p, int Lq, int Lk, int batch, int offset,
                        float scale, void *stream);

/* ------------------------------------------------------------------------
 * Fused causal self-attention of the decoder composition (TBIK summary
 * page, "technical framework").  For every sequence b < batch and head
 * h < heads it writes exactly the bits of the unfused composition
 *   S = tbik_gemm(Q_bh, K_bh)                      (fp32, K = head_dim)
 *   P = tbik_softmax_causal(S, offset 0, scale)    (bf16)
 *   O_bh = bf16(tbik_gemm(P, Vt_bh))
 * without writing S or P to memory.
 *  Q, K   [batch*L, ldq / ldk] bf16: token t = b*L + i; head h in columns
 *         [h*128, h*128 + 128).
 *  Vt     [heads*128, ldvt] bf16: V transposed, row h*128 + n, column
 *         b*L + j (ldvt >= batch*L).
 *  O      [batch*L, ldo] bf16, same layout as Q.
 *  head_dim must be 128; L one of 64, 128, 256, 512; strides multiples of 8
 *  and Q, K, Vt 16-byte aligned.
 * ---------------------------------------------------------------------- */
int tbik_attention_causal(const tbik_bf16 *Q, int64_t ldq, const tbik_bf16 *K, int64_t ldk,
                          const tbik_bf16 *Vt, int64_t ldvt, tbik_bf16 *O, int64_t ldo, int L,
                          int heads, int head_dim, int batch, float scale, void *stream);

/* ------------------------------------------------------------------------
 * Row gather, the embedding lookup of the decoder composition (TBIK summary
 * page, "technical framework": the invariant kernels inside a full model):
 *   out[i, :] = table[idx[i], :]  for i < n; an index outside [0, rows)
 *   gives a zero row.  A copy: no arithmetic.
 *  table  [rows, cols] bf16, row stride ld_table.
 *  idx    [n] int32 device array.
 *  out    [n, cols] bf16, row stride ld_out.
 * ---------------------------------------------------------------------- */
int tbik_gather_rows(const tbik_bf16 *table, int64_t ld_table, int rows, const int32_t *idx,
                     int n, int cols, tbik_bf16 *out, int64_t ld_out, void *stream);

/* ------------------------------------------------------------------------
 * The library's fp32/bf16 primitives applied elementwise (for checking):
 *  op 0: EXP(x)   op 1: LOG(x)   op 2: bf16 round-to-nearest-even of x,
 *  widened back to fp32 (a NaN gives a quiet NaN of unspecified payload)
 *  op 3: g / (1 + EXP(-g)) with g = bf16(x): the SwiGLU gate activation of
 *  a bf16 gate, its division correctly rounded.
 *  x, y: [n] fp32 device arrays.
 * ---------------------------------------------------------------------- */
enum { TBIK_PRIM_EXP = 0, TBIK_PRIM_LOG = 1, TBIK_PRIM_BF16 = 2, TBIK_PRIM_SILU = 3 };

int tbik_primitive(int op, const float *x, float *y, int64_t n, void *stream);

/* ========================================================================
 * Training side ([TBIK] Abstract: the trainer -- FSDP, TP = 1 -- and the
 * inference engine must give bit-identical results; [ROUND] "three nodes":
 * fp32 intermediates, one bf16 rounding per output).  The pages give no
 * backward formulas: each backward below is the derivative of the forward
 * definition above, in fp32, in the order written.  Sums over tokens are
 * TREE over 64-token leaves, so a data-parallel split of the tokens into dp
 * ranks (dp in {1,2,4,8} dividing T of the leaf count) is a split at aligned
 * groups, and the result is bit-identical for every dp; dp simulates that
 * split on one GPU (shard nodes, then the top of the tree).
 * ====================================================================== */

/* y = x^T: x [rows, cols] bf16 (row stride ldx) -> y [cols, rows] bf16
 * (row stride ldy).  Bits are copied.  rows <= 4194240. */
int tbik_transpose_bf16(const tbik_bf16 *x, int64_t ldx, tbik_bf16 *y, int64_t ldy, int rows,
                        int cols, void *stream);

/* Input gradient of Y = X W^T:  dX = dY W, i.e. dX[m,k] = TREE_n(dY[m,n] W[n,k])
 * over the N/64 leaves of n (the forward GEMM's tree with N as the reduced
 * dimension).  dY [M,N] (ld_dy), W [N,K] (ldw), dX [M,K] fp32 (ld_dx) and/or
 * dX_bf16 (same ld).  N must be a positive multiple of 64.  W is transposed
 * into ws first: ws_bytes >= tbik_gemm_dgrad_workspace_bytes(M, N, K),
 * ws 16-byte aligned, device memory owned by the caller. */
size_t tbik_gemm_dgrad_workspace_bytes(int M, int N, int K);
int tbik_gemm_dgrad(const tbik_bf16 *dY, int64_t ld_dy, const tbik_bf16 *W, int64_t ldw, float *dX,
                    int64_t ld_dx, tbik_bf16 *dX_bf16, int M, int N, int K, int leaf_mode,
                    void *ws, size_t ws_bytes, void *stream);

/* Weight gradient of Y = X W^T:  dW = dY^T X, i.e. dW[n,k] = TREE_m(dY[m,n] X[m,k])
 * over the M/64 token leaves.  dY [M,N] (ld_dy), X [M,K] (ldx), dW [N,K] fp32
 * (ld_dw).  M must be a positive multiple of 64; dp in {1,2,4,8} divides
 * T(M/64) (else TBIK_ERR_TP).  ws (>= tbik_gemm_wgrad_workspace_bytes) holds
 * dY^T [N,M] bf16, then X^T [K,M] bf16, each at a 256-byte boundary, then
 * with dp > 1 the dp shard partials [dp][N][K] fp32 (kept after return). */
size_t tbik_gemm_wgrad_workspace_bytes(int M, int N, int K, int dp);
int tbik_gemm_wgrad(const tbik_bf16 *dY, int64_t ld_dy, const tbik_bf16 *X, int64_t ldx, float *dW,
                    int64_t ld_dw, int M, int N, int K, int dp, int leaf_mode, void *ws,
                    size_t ws_bytes, void *stream);

/* RoPE backward: the adjoint of the rotation, the rotation by -angle:
 *   dx[i] = bf16(dy[i]*c + dy[i+d/2]*s),  dx[i+d/2] = bf16(dy[i+d/2]*c - dy[i]*s),
 * each product rounded to fp32 separately.  Layout and limits as tbik_rope;
 * dx == dy (in place) is allowed. */
int tbik_rope_backward(const tbik_bf16 *dy, tbik_bf16 *dx, const int32_t *pos,
                       const float *cos_tab, const float *sin_tab, int T, int heads, int head_dim,
                       int64_t ld_token, int max_pos, void *stream);

/* SwiGLU backward for out = silu(g) * u:
 *   den = 1 + EXP(-g);  sig = 1/den;  silu = g/den   (divisions correctly rounded)
 *   dup   = bf16(dout * silu)
 *   dgate = bf16((dout * u) * (sig * (1 + g * (1 - sig)))).
 *  gate, up, dout, dgate, dup  [rows, cols] bf16 with their own row strides. */
int tbik_swiglu_backward(const tbik_bf16 *gate, const tbik_bf16 *up, const tbik_bf16 *dout,
                         tbik_bf16 *dgate, tbik_bf16 *dup, int rows, int cols, int64_t ld_gate,
                         int64_t ld_up, int64_t ld_dout, int64_t ld_dgate, int64_t ld_dup,
                         void *stream);

/* Residual RMSNorm backward.  The forward (tbik_rmsnorm_residual) is
 * recomputed: h = x + r, rstd from TREE_j(h_j*h_j) with the same bits.  Given
 * dy = dL/dy and dr = dL/dr_out (NULL = zero), per row:
 *   g_j = dy_j * w_j;  dot = TREE_j(g_j * h_j);  c = (dot * ((rstd*rstd)*rstd)) / H;
 *   dh_j = bf16(((rstd * g_j) - (c * h_j)) + dr_j)          (= dL/dx = dL/dr);
 * and, when dw is not NULL, the weight gradient over the rows (tokens):
 *   leaf b of column j = sum over rows 64b..64b+63, in row order from +0, of
 *   dy_ij * (h_ij * rstd_i);  dw_j = TREE over the leaves as dp shards.
 * rows must then be a positive multiple of 64 and dp divide T(rows/64).
 * H is 1 .. 65536, any value, as for the forward.
 * ws (fp32, >= tbik_rmsnorm_backward_workspace_bytes) holds, in floats:
 * rstd per row (rows rounded up to a multiple of 64), then with dw the
 * (rows/64) x H leaves and the dp x H shard nodes (kept after return). */
size_t tbik_rmsnorm_backward_workspace_bytes(int rows, int H, int dp, int want_dw);
int tbik_rmsnorm_backward(const tbik_bf16 *x, const tbik_bf16 *r, const tbik_bf16 *w,
                          const tbik_bf16 *dy, const tbik_bf16 *dr, tbik_bf16 *dh, float *dw,
                          int rows, int H, int64_t ld, float eps, int dp, float *ws,
                          size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * tbik_gemm without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc).  Same arguments, results and bits as tbik_gemm
 * given a workspace of tbik_gemm_workspace_bytes(M, N, K): the split-K node
 * partials go to a file-scope device array of tbik_gemm_noalloc_max_bytes()
 * = 16 MiB held by every GPU the library runs on until the process ends.
 * The call allocates nothing.  A shape whose workspace would exceed that
 * size returns TBIK_ERR_WORKSPACE before any launch (shapes needing no
 * workspace always run).  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (concurrent streams, or threads
 * without ordering) race and must not be issued.  The array's device
 * address is resolved on the first call made with a given device current.
 * ---------------------------------------------------------------------- */
size_t tbik_gemm_noalloc_max_bytes(void);
int tbik_gemm_noalloc(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw, float *C,
                      int64_t ldc, tbik_bf16 *C_bf16, int M, int N, int K, int leaf_mode,
                      void *stream);

/* ------------------------------------------------------------------------
 * Ceiling microbenchmarks.  Not part of the method: the attainable rates of
 * this GPU, so that every roofline fraction can be stated against both the
 * published peak and what the chip sustains (a pure matrix-core loop and
 * non-temporal HBM streams over buffers far larger than the last-level
 * cache).  Results are timed by the caller on `stream`.
 *
 * tbik_bench_mfma: `blocks` workgroups of 8 waves, each wave running 8
 *   independent chains of `iters` v_mfma_f32_16x16x32_bf16 from registers.
 *   seed: >= 2048 bytes of device memory (16-byte aligned) holding the
 *   operands; out: blocks * 512 floats (one per thread, keeps the chains
 *   live).  tbik_bench_mfma_flops gives the flops of one launch (0 for
 *   invalid arguments).
 * tbik_bench_hbm_read: `blocks` workgroups of 256 threads stream `bytes`
 *   (a positive multiple of 16) of buf with non-temporal 16-byte loads;
 *   out: blocks * 256 unsigned (an xor of what each thread read).
 * tbik_bench_hbm_copy: src -> dst, `bytes` (multiple of 16), non-temporal
 *   16-byte loads and stores; the buffers must not overlap.
 * tbik_bench_copy_lds: the GEMM ring's operand copy without the MFMAs.
 *   `blocks` workgroups of 8 waves (128 KB of LDS each) each move `stages`
 *   stages of 32 KB from buf into a 4-slot LDS ring with 16-byte-per-lane
 *   global->LDS buffer loads, 3 stages ahead, one barrier per stage.  The
 *   stages are read cyclically from the first `window_bytes` of buf (a
 *   multiple of 32768, at most 2^31 - 32768), workgroup b starting at stage
 *   7b.  Bytes moved = blocks * stages * 32768.  A window that fits one XCD's
 *   L2 (4 MB) measures the L2 -> LDS rate; larger ones, the last-level cache
 *   or HBM through the same path.  out: blocks * 512 unsigned.
 * Errors: TBIK_ERR_NULL, TBIK_ERR_SHAPE (sizes out of range),
 * TBIK_ERR_ALIGN (pointers not 16-byte aligned), TBIK_ERR_LAUNCH.
 * ---------------------------------------------------------------------- */
int64_t tbik_bench_mfma_flops(int blocks, int iters);
int tbik_bench_mfma(const void *seed, float *out, int blocks, int iters, void *stream);
int tbik_bench_hbm_read(const void *buf, int64_t bytes, unsigned *out, int blocks, void *stream);
int tbik_bench_hbm_copy(const void *src, void *dst, int64_t bytes, int blocks, void *stream);
int tbik_bench_copy_lds(const void *buf, int64_t window_bytes, int stages, unsigned *out,
                        int blocks, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* TBIK_H */
