// tbik_abi.hip -- the extern "C" entry points of libtbik.so.
//
// Host-side validation happens before any HIP call; an invalid call
// launches nothing and returns a TBIK_ERR_* code.  No entry point allocates
// memory.  The only state kept between calls is the per-device address of
// tbik_gemm_noalloc's scratch array, resolved once.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/tbik.h"
#include "tbik_device.h"
#include "tbik_internal.h"

using tbik::GemmCall;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned(const void *p, unsigned a) { return ((uintptr_t)p & (a - 1u)) == 0; }
bool ld_ok(int64_t ld) { return ld > 0 && (ld % 8) == 0; }
hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }
bool tp_ok(int tp) { return tp == 1 || tp == 2 || tp == 4 || tp == 8; }

// Common checks of a GEMM call (both modes).
int check_gemm(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw, const float *C,
               int64_t ldc, const tbik_bf16 *Cb, int M, int N, int K, int leaf_mode) {
  if (!A || !W || (!C && !Cb)) return TBIK_ERR_NULL;
  if (M < 0 || N < 0 || K <= 0 || (K % 64) != 0) return TBIK_ERR_SHAPE;
  if (lda < K || ldw < K || ldc < N) return TBIK_ERR_SHAPE;
  if (!ld_ok(lda) || !ld_ok(ldw)) return TBIK_ERR_ALIGN;
  if (!aligned16(A) || !aligned16(W) || (C && !aligned(C, 4)) || (Cb && !aligned(Cb, 2)))
    return TBIK_ERR_ALIGN;
  if (leaf_mode != TBIK_LEAF_MFMA && leaf_mode != TBIK_LEAF_SCALAR) return TBIK_ERR_ARG;
  const int nb = K / 64;
  if (nb / tbik::tree_T(nb) > tbik::kMaxGroupLeaves) return TBIK_ERR_SHAPE;
  return TBIK_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of tbik_gemm_noalloc: the split-K node partials live in this
// file-scope device array instead of a caller's workspace.  Each GPU the
// library runs on holds its own copy until the process ends; in host code
// the name is only a stand-in, so its device address is resolved once per
// device with hipGetSymbolAddress and only that address is ever passed on.
// ---------------------------------------------------------------------------
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;   // 16 MiB
static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (resolved on the first
// call made with that device current).
int scratch_for_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TBIK_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return TBIK_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TBIK_OK;
}

}  // namespace

extern "C" {

int tbik_version(void) { return 1 * 10000 + 0 * 100 + 0; }

const char *tbik_strerror(int code) {
  switch (code) {
    case TBIK_OK: return "ok";
    case TBIK_ERR_NULL: return "a required pointer is NULL";
    case TBIK_ERR_SHAPE: return "invalid shape (negative size, K not a positive multiple of 64, "
                                "leading dimension too small, or size beyond the supported range)";
    case TBIK_ERR_TP: return "tp must be 1, 2, 4 or 8 and divide the tree's group count T";
    case TBIK_ERR_ALIGN: return "pointers must be 16-byte aligned and leading dimensions multiples of 8";
    case TBIK_ERR_WORKSPACE: return "workspace missing or too small";
    case TBIK_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case TBIK_ERR_ARG: return "argument out of range";
  }
  return "unknown error code";
}

int tbik_tree_groups(int64_t n) { return n <= 0 ? 0 : tbik::tree_T(n); }

size_t tbik_gemm_workspace_bytes(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0 || (K % 64) != 0) return 0;
  const int p = tbik::gemm_split_parts(M, N, K, 1, TBIK_LEAF_MFMA);
  return p > 1 ? (size_t)p * (size_t)M * (size_t)N * sizeof(float) : 0;
}

int tbik_gemm(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw, float *C,
              int64_t ldc, tbik_bf16 *C_bf16, int M, int N, int K, int leaf_mode, float *ws,
              size_t ws_bytes, void *stream) {
  int rc = check_gemm(A, lda, W, ldw, C, ldc, C_bf16, M, N, K, leaf_mode);
  if (rc) return rc;
  if (M == 0 || N == 0) return TBIK_OK;
  const int p = tbik::gemm_split_parts(M, N, K, 1, leaf_mode);
  // Split K into p aligned tree nodes only when the caller's workspace holds
  // them; otherwise (or when p == 1) one launch computes the whole tree.
  // Both give the same bits: the split is at node boundaries.
  if (p > 1 && ws && aligned(ws, 16) &&
      ws_bytes >= (size_t)p * (size_t)M * (size_t)N * sizeof(float)) {
    GemmCall c{};
    c.A = A; c.lda = lda; c.strideA = 0;
    c.W = W; c.ldw = ldw; c.strideW = 0;
    c.C = ws; c.Cb = nullptr; c.ldc = N; c.strideC = 0; c.part_stride = (int64_t)M * N;
    c.M = M; c.N = N; c.K = K; c.batch = 1; c.parts = p; c.leaf_mode = leaf_mode;
    rc = tbik::launch_gemm(c, as_stream(stream));
    if (rc) return rc;
    return tbik::launch_tree_combine(ws, p, C, ldc, C_bf16, M, N, as_stream(stream));
  }
  return tbik_gemm_strided_batched(A, lda, 0, W, ldw, 0, C, ldc, 0, C_bf16, M, N, K, 1, leaf_mode,
                                   stream);
}

size_t tbik_gemm_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

int tbik_gemm_noalloc(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw, float *C,
                      int64_t ldc, tbik_bf16 *C_bf16, int M, int N, int K, int leaf_mode,
                      void *stream) {
  int rc = check_gemm(A, lda, W, ldw, C, ldc, C_bf16, M, N, K, leaf_mode);
  if (rc) return rc;
  if (M == 0 || N == 0) return TBIK_OK;
  const size_t need = leaf_mode == TBIK_LEAF_MFMA ? tbik_gemm_workspace_bytes(M, N, K) : 0;
  if (need > kNoallocScratchBytes) return TBIK_ERR_WORKSPACE;
  void *ws = nullptr;
  if (need > 0) {
    rc = scratch_for_current_device(&ws);
    if (rc) return rc;
  }
  return tbik_gemm(A, lda, W, ldw, C, ldc, C_bf16, M, N, K, leaf_mode, static_cast<float *>(ws),
                   need, stream);
}

int tbik_gemm_strided_batched(const tbik_bf16 *A, int64_t lda, int64_t strideA,
                              const tbik_bf16 *W, int64_t ldw, int64_t strideW, float *C,
                              int64_t ldc, int64_t strideC, tbik_bf16 *C_bf16, int M, int N,
                              int K, int batch, int leaf_mode, void *stream) {
  int rc = check_gemm(A, lda, W, ldw, C, ldc, C_bf16, M, N, K, leaf_mode);
  if (rc) return rc;
  if (batch < 0 || batch > 65535) return TBIK_ERR_SHAPE;
  if (strideA < 0 || strideW < 0 || strideC < 0) return TBIK_ERR_SHAPE;
  if ((strideA % 8) || (strideW % 8)) return TBIK_ERR_ALIGN;
  if (M == 0 || N == 0 || batch == 0) return TBIK_OK;
  GemmCall c{};
  c.A = A; c.lda = lda; c.strideA = strideA;
  c.W = W; c.ldw = ldw; c.strideW = strideW;
  c.C = C; c.Cb = C_bf16; c.ldc = ldc; c.strideC = strideC; c.part_stride = 0;
  c.M = M; c.N = N; c.K = K; c.batch = batch; c.parts = 1; c.leaf_mode = leaf_mode;
  return tbik::launch_gemm(c, as_stream(stream));
}

size_t tbik_gemm_tpsim_workspace_bytes(int M, int N, int K, int tp) {
  if (M < 0 || N < 0 || tp < 1) return 0;
  (void)K;
  return (size_t)tp * (size_t)M * (size_t)N * sizeof(float);
}

int tbik_gemm_tpsim(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw, float *C,
                    int64_t ldc, tbik_bf16 *C_bf16, int M, int N, int K, int tp, int leaf_mode,
                    float *ws, size_t ws_bytes, void *stream) {
  int rc = check_gemm(A, lda, W, ldw, C, ldc, C_bf16, M, N, K, leaf_mode);
  if (rc) return rc;
  const int T = tbik::tree_T(K / 64);
  if (!tp_ok(tp) || (T % tp) != 0) return TBIK_ERR_TP;
  if (M == 0 || N == 0) return TBIK_OK;
  if (!ws) return TBIK_ERR_WORKSPACE;
  if (ws_bytes < tbik_gemm_tpsim_workspace_bytes(M, N, K, tp)) return TBIK_ERR_WORKSPACE;
  if (!aligned(ws, 4)) return TBIK_ERR_ALIGN;
  GemmCall c{};
  c.A = A; c.lda = lda; c.strideA = 0;
  c.W = W; c.ldw = ldw; c.strideW = 0;
  c.C = ws; c.Cb = nullptr; c.ldc = N; c.strideC = 0; c.part_stride = (int64_t)M * N;
  c.M = M; c.N = N; c.K = K; c.batch = 1; c.parts = tp; c.leaf_mode = leaf_mode;
  rc = tbik::launch_gemm(c, as_stream(stream));
  if (rc) return rc;
  return tbik::launch_tree_combine(ws, tp, C, ldc, C_bf16, M, N, as_stream(stream));
}

int tbik_gemm_tp_partials(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw,
                          float *ws, size_t ws_bytes, int M, int N, int K, int tp, int leaf_mode,
                          void *stream) {
  int rc = check_gemm(A, lda, W, ldw, ws, N, nullptr, M, N, K, leaf_mode);
  if (rc) return rc;
  const int T = tbik::tree_T(K / 64);
  if (!tp_ok(tp) || (T % tp) != 0) return TBIK_ERR_TP;
  if (M == 0 || N == 0) return TBIK_OK;
  if (ws_bytes < tbik_gemm_tpsim_workspace_bytes(M, N, K, tp)) return TBIK_ERR_WORKSPACE;
  GemmCall c{};
  c.A = A; c.lda = lda; c.strideA = 0;
  c.W = W; c.ldw = ldw; c.strideW = 0;
  c.C = ws; c.Cb = nullptr; c.ldc = N; c.strideC = 0; c.part_stride = (int64_t)M * N;
  c.M = M; c.N = N; c.K = K; c.batch = 1; c.parts = tp; c.leaf_mode = leaf_mode;
  return tbik::launch_gemm(c, as_stream(stream));
}

int tbik_gemm_shard(const tbik_bf16 *A_t, int64_t lda, const tbik_bf16 *W_t, int64_t ldw,
                    float *P, int64_t ldp, int M, int N, int K_total, int tp, int leaf_mode,
                    void *stream) {
  if (!tp_ok(tp) || K_total <= 0 || (K_total % 64) != 0) return !tp_ok(tp) ? TBIK_ERR_TP
                                                                           : TBIK_ERR_SHAPE;
  const int T = tbik::tree_T(K_total / 64);
  if ((T % tp) != 0) return TBIK_ERR_TP;
  const int K = K_total / tp;
  int rc = check_gemm(A_t, lda, W_t, ldw, P, ldp, nullptr, M, N, K, leaf_mode);
  if (rc) return rc;
  const int nb = K_total / 64;
  if (nb / T > tbik::kMaxGroupLeaves) return TBIK_ERR_SHAPE;
  if (M == 0 || N == 0) return TBIK_OK;
  GemmCall c{};
  c.A = A_t; c.lda = lda; c.strideA = 0;
  c.W = W_t; c.ldw = ldw; c.strideW = 0;
  c.C = P; c.Cb = nullptr; c.ldc = ldp; c.strideC = 0; c.part_stride = 0;
  c.M = M; c.N = N; c.K = K; c.batch = 1; c.parts = 1; c.leaf_mode = leaf_mode;
  c.tree_leaves = nb; c.shard_of = tp;
  return tbik::launch_gemm(c, as_stream(stream));
}

int tbik_tree_combine(const float *ws, int tp, float *C, int64_t ldc, tbik_bf16 *C_bf16, int M,
                      int N, void *stream) {
  if (!ws || (!C && !C_bf16)) return TBIK_ERR_NULL;
  if (!tp_ok(tp)) return TBIK_ERR_TP;
  if (M < 0 || N < 0 || ldc < N) return TBIK_ERR_SHAPE;
  if (!aligned(ws, 4) || (C && !aligned(C, 4)) || (C_bf16 && !aligned(C_bf16, 2)))
    return TBIK_ERR_ALIGN;
  if (M == 0 || N == 0) return TBIK_OK;
  return tbik::launch_tree_combine(ws, tp, C, ldc, C_bf16, M, N, as_stream(stream));
}

static bool rounding_ok(int rounding) {
  return rounding == TBIK_ROUND_ONCE || rounding == TBIK_ROUND_EACH_OP;
}

int tbik_rmsnorm_residual(const tbik_bf16 *x, const tbik_bf16 *r, const tbik_bf16 *w,
                          tbik_bf16 *y, tbik_bf16 *r_out, int rows, int H, int64_t ld, float eps,
                          void *stream) {
  return tbik_rmsnorm_residual_ex(x, r, w, y, r_out, rows, H, ld, eps, TBIK_ROUND_ONCE, stream);
}

int tbik_rmsnorm_residual_ex(const tbik_bf16 *x, const tbik_bf16 *r, const tbik_bf16 *w,
                             tbik_bf16 *y, tbik_bf16 *r_out, int rows, int H, int64_t ld,
                             float eps, int rounding, void *stream) {
  if (!x || !r || !w || !y) return TBIK_ERR_NULL;
  if (!rounding_ok(rounding)) return TBIK_ERR_ARG;
  if (rows < 0 || H < 1 || H > 65536 || ld < H) return TBIK_ERR_SHAPE;
  if (!(eps >= 0.0f) || isinf(eps)) return TBIK_ERR_ARG;
  if (!aligned(x, 2) || !aligned(r, 2) || !aligned(w, 2) || !aligned(y, 2) ||
      (r_out && !aligned(r_out, 2)))
    return TBIK_ERR_ALIGN;
  if (rows == 0) return TBIK_OK;
  return tbik::launch_rmsnorm_residual(x, r, w, y, r_out, rows, H, ld, eps, rounding,
                                       as_stream(stream));
}

int tbik_rope(const tbik_bf16 *x, tbik_bf16 *y, const int32_t *pos, const float *cos_tab,
              const float *sin_tab, int T, int heads, int head_dim, int64_t ld_token,
              int max_pos, void *stream) {
  return tbik_rope_ex(x, y, pos, cos_tab, sin_tab, T, heads, head_dim, ld_token, max_pos,
                      TBIK_ROUND_ONCE, stream);
}

int tbik_rope_ex(const tbik_bf16 *x, tbik_bf16 *y, const int32_t *pos, const float *cos_tab,
                 const float *sin_tab, int T, int heads, int head_dim, int64_t ld_token,
                 int max_pos, int rounding, void *stream) {
  if (!x || !y || !pos || !cos_tab || !sin_tab) return TBIK_ERR_NULL;
  if (!rounding_ok(rounding)) return TBIK_ERR_ARG;
  if (T < 0 || heads < 1 || max_pos < 1) return TBIK_ERR_SHAPE;
  if (head_dim < 2 || head_dim > 1024 || (head_dim % 8) != 0) return TBIK_ERR_SHAPE;
  if (ld_token < (int64_t)heads * head_dim) return TBIK_ERR_SHAPE;
  if (!ld_ok(ld_token)) return TBIK_ERR_ALIGN;
  if (!aligned16(x) || !aligned16(y) || !aligned16(cos_tab) || !aligned16(sin_tab) ||
      ((uintptr_t)pos & 3u))
    return TBIK_ERR_ALIGN;
  if (T == 0) return TBIK_OK;
  return tbik::launch_rope(x, y, pos, cos_tab, sin_tab, T, heads, head_dim, ld_token, max_pos,
                           rounding, as_stream(stream));
}

int tbik_rope_table(double theta, int head_dim, int max_pos, float *cos_tab, float *sin_tab) {
  if (!cos_tab || !sin_tab) return TBIK_ERR_NULL;
  if (!(theta > 0.0) || head_dim < 2 || (head_dim % 2) || max_pos < 1) return TBIK_ERR_ARG;
  const int half = head_dim / 2;
  for (int i = 0; i < half; ++i) {
    // theta^(-2i/d) in binary64, then the angle p * freq in binary64
    const double freq = pow(theta, -(2.0 * i) / (double)head_dim);
    for (int p = 0; p < max_pos; ++p) {
      const double ang = (double)p * freq;
      cos_tab[(int64_t)p * half + i] = (float)cos(ang);
      sin_tab[(int64_t)p * half + i] = (float)sin(ang);
    }
  }
  return TBIK_OK;
}

int tbik_swiglu(const tbik_bf16 *gate, const tbik_bf16 *up, tbik_bf16 *out, int rows, int cols,
                int64_t ld_gate, int64_t ld_up, int64_t ld_out, void *stream) {
  return tbik_swiglu_ex(gate, up, out, rows, cols, ld_gate, ld_up, ld_out, TBIK_ROUND_ONCE,
                        stream);
}

int tbik_gemm_swiglu(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W_gu, int64_t ldw,
                     tbik_bf16 *H, int64_t ldh, int M, int F, int K, int rounding, void *stream) {
  if (!H) return TBIK_ERR_NULL;
  if (F <= 0 || (F % 16) != 0 || F > (1 << 29) || ldh < F) return TBIK_ERR_SHAPE;
  if (!rounding_ok(rounding)) return TBIK_ERR_ARG;
  int rc = check_gemm(A, lda, W_gu, ldw, nullptr, 2 * (int64_t)F, H, M, 2 * F, K, TBIK_LEAF_MFMA);
  if (rc) return rc;
  if (M == 0) return TBIK_OK;
  tbik::GemmCall c{};
  c.A = A; c.lda = lda; c.strideA = 0;
  c.W = W_gu; c.ldw = ldw; c.strideW = 0;
  c.C = nullptr; c.Cb = nullptr; c.ldc = 2 * (int64_t)F; c.strideC = 0; c.part_stride = 0;
  c.M = M; c.N = 2 * F; c.K = K; c.batch = 1; c.parts = 1; c.leaf_mode = TBIK_LEAF_MFMA;
  c.H = H; c.ldh = ldh; c.glu = rounding == TBIK_ROUND_EACH_OP ? 2 : 1;
  return tbik::launch_gemm(c, as_stream(stream));
}

int tbik_swiglu_ex(const tbik_bf16 *gate, const tbik_bf16 *up, tbik_bf16 *out, int rows,
                   int cols, int64_t ld_gate, int64_t ld_up, int64_t ld_out, int rounding,
                   void *stream) {
  if (!gate || !up || !out) return TBIK_ERR_NULL;
  if (!rounding_ok(rounding)) return TBIK_ERR_ARG;
  if (rows < 0 || cols < 0 || ld_gate < cols || ld_up < cols || ld_out < cols)
    return TBIK_ERR_SHAPE;
  if (!aligned(gate, 2) || !aligned(up, 2) || !aligned(out, 2)) return TBIK_ERR_ALIGN;
  if (rows == 0 || cols == 0) return TBIK_OK;
  return tbik::launch_swiglu(gate, up, out, rows, cols, ld_gate, ld_up, ld_out, rounding,
                             as_stream(stream));
}

// ---------------------------------------------------------------- training side

int tbik_transpose_bf16(const tbik_bf16 *x, int64_t ldx, tbik_bf16 *y, int64_t ldy, int rows,
                        int cols, void *stream) {
  if (!x || !y) return TBIK_ERR_NULL;
  if (rows < 0 || cols < 0 || rows > 4194240 || ldx < cols || ldy < rows) return TBIK_ERR_SHAPE;
  if (!aligned(x, 2) || !aligned(y, 2)) return TBIK_ERR_ALIGN;
  if (rows == 0 || cols == 0) return TBIK_OK;
  return tbik::launch_transpose_bf16(x, ldx, y, ldy, rows, cols, as_stream(stream));
}

static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

size_t tbik_gemm_dgrad_workspace_bytes(int M, int N, int K) {
  if (M < 0 || N <= 0 || K <= 0) return 0;
  return round256((size_t)K * (size_t)N * 2);
}

int tbik_gemm_dgrad(const tbik_bf16 *dY, int64_t ld_dy, const tbik_bf16 *W, int64_t ldw, float *dX,
                    int64_t ld_dx, tbik_bf16 *dX_bf16, int M, int N, int K, int leaf_mode,
                    void *ws, size_t ws_bytes, void *stream) {
  if (!dY || !W || (!dX && !dX_bf16)) return TBIK_ERR_NULL;
  if (M < 0 || K < 0 || N <= 0 || (N % 64) != 0 || ldw < K) return TBIK_ERR_SHAPE;
  if (!aligned(W, 2)) return TBIK_ERR_ALIGN;
  if (M == 0 || K == 0) return TBIK_OK;
  if (!ws) return TBIK_ERR_WORKSPACE;
  if (!aligned16(ws)) return TBIK_ERR_ALIGN;
  if (ws_bytes < tbik_gemm_dgrad_workspace_bytes(M, N, K)) return TBIK_ERR_WORKSPACE;
  tbik_bf16 *Wt = static_cast<tbik_bf16 *>(ws);                  // [K, N]
  // the GEMM's own checks on the transposed layout, before anything runs
  int rc = check_gemm(dY, ld_dy, Wt, N, dX, ld_dx, dX_bf16, M, K, N, leaf_mode);
  if (rc) return rc;
  rc = tbik::launch_transpose_bf16(W, ldw, Wt, N, N, K, as_stream(stream));
  if (rc) return rc;
  return tbik_gemm_strided_batched(dY, ld_dy, 0, Wt, N, 0, dX, ld_dx, 0, dX_bf16, M, K, N, 1,
                                   leaf_mode, stream);
}

size_t tbik_gemm_wgrad_workspace_bytes(int M, int N, int K, int dp) {
  if (M <= 0 || N < 0 || K < 0 || dp < 1) return 0;
  size_t b = round256((size_t)N * (size_t)M * 2) + round256((size_t)K * (size_t)M * 2);
  if (dp > 1) b += (size_t)dp * (size_t)N * (size_t)K * sizeof(float);
  return b;
}

int tbik_gemm_wgrad(const tbik_bf16 *dY, int64_t ld_dy, const tbik_bf16 *X, int64_t ldx, float *dW,
                    int64_t ld_dw, int M, int N, int K, int dp, int leaf_mode, void *ws,
                    size_t ws_bytes, void *stream) {
  if (!dY || !X || !dW) return TBIK_ERR_NULL;
  if (M <= 0 || (M % 64) != 0 || N < 0 || K < 0 || ld_dy < N || ldx < K || ld_dw < K)
    return TBIK_ERR_SHAPE;
  if (M > 4194240) return TBIK_ERR_SHAPE;
  if (!tp_ok(dp) || (tbik::tree_T(M / 64) % dp) != 0) return TBIK_ERR_TP;
  if (!aligned(dY, 2) || !aligned(X, 2) || !aligned(dW, 4)) return TBIK_ERR_ALIGN;
  if (leaf_mode != TBIK_LEAF_MFMA && leaf_mode != TBIK_LEAF_SCALAR) return TBIK_ERR_ARG;
  const int nb = M / 64;
  if (nb / tbik::tree_T(nb) > tbik::kMaxGroupLeaves) return TBIK_ERR_SHAPE;
  if (N == 0 || K == 0) return TBIK_OK;
  if (!ws) return TBIK_ERR_WORKSPACE;
  if (!aligned16(ws)) return TBIK_ERR_ALIGN;
  if (ws_bytes < tbik_gemm_wgrad_workspace_bytes(M, N, K, dp)) return TBIK_ERR_WORKSPACE;
  char *base = static_cast<char *>(ws);
  tbik_bf16 *dYt = reinterpret_cast<tbik_bf16 *>(base);                       // [N, M]
  tbik_bf16 *Xt = reinterpret_cast<tbik_bf16 *>(base + round256((size_t)N * M * 2));  // [K, M]
  float *parts = reinterpret_cast<float *>(base + round256((size_t)N * M * 2) +
                                           round256((size_t)K * M * 2));
  hipStream_t s = as_stream(stream);
  int rc = tbik::launch_transpose_bf16(dY, ld_dy, dYt, M, M, N, s);
  if (rc) return rc;
  rc = tbik::launch_transpose_bf16(X, ldx, Xt, M, M, K, s);
  if (rc) return rc;
  if (dp == 1)
    return tbik_gemm_strided_batched(dYt, M, 0, Xt, M, 0, dW, ld_dw, 0, nullptr, N, K, M, 1,
                                     leaf_mode, stream);
  return tbik_gemm_tpsim(dYt, M, Xt, M, dW, ld_dw, nullptr, N, K, M, dp, leaf_mode, parts,
                         (size_t)dp * N * K * sizeof(float), stream);
}

int tbik_rope_backward(const tbik_bf16 *dy, tbik_bf16 *dx, const int32_t *pos,
                       const float *cos_tab, const float *sin_tab, int T, int heads, int head_dim,
                       int64_t ld_token, int max_pos, void *stream) {
  if (!dy || !dx || !pos || !cos_tab || !sin_tab) return TBIK_ERR_NULL;
  if (T < 0 || heads < 1 || max_pos < 1) return TBIK_ERR_SHAPE;
  if (head_dim < 2 || head_dim > 1024 || (head_dim % 8) != 0) return TBIK_ERR_SHAPE;
  if (ld_token < (int64_t)heads * head_dim) return TBIK_ERR_SHAPE;
  if (!ld_ok(ld_token)) return TBIK_ERR_ALIGN;
  if (!aligned16(dy) || !aligned16(dx) || !aligned16(cos_tab) || !aligned16(sin_tab) ||
      ((uintptr_t)pos & 3u))
    return TBIK_ERR_ALIGN;
  if (T == 0) return TBIK_OK;
  return tbik::launch_rope_backward(dy, dx, pos, cos_tab, sin_tab, T, heads, head_dim, ld_token,
                                    max_pos, as_stream(stream));
}

int tbik_swiglu_backward(const tbik_bf16 *gate, const tbik_bf16 *up, const tbik_bf16 *dout,
                         tbik_bf16 *dgate, tbik_bf16 *dup, int rows, int cols, int64_t ld_gate,
                         int64_t ld_up, int64_t ld_dout, int64_t ld_dgate, int64_t ld_dup,
                         void *stream) {
  if (!gate || !up || !dout || !dgate || !dup) return TBIK_ERR_NULL;
  if (rows < 0 || cols < 0 || ld_gate < cols || ld_up < cols || ld_dout < cols ||
      ld_dgate < cols || ld_dup < cols)
    return TBIK_ERR_SHAPE;
  if (!aligned(gate, 2) || !aligned(up, 2) || !aligned(dout, 2) || !aligned(dgate, 2) ||
      !aligned(dup, 2))
    return TBIK_ERR_ALIGN;
  if (rows == 0 || cols == 0) return TBIK_OK;
  return tbik::launch_swiglu_backward(gate, up, dout, dgate, dup, rows, cols, ld_gate, ld_up,
                                      ld_dout, ld_dgate, ld_dup, as_stream(stream));
}

size_t tbik_rmsnorm_backward_workspace_bytes(int rows, int H, int dp, int want_dw) {
  if (rows < 0 || H < 1 || dp < 1) return 0;
  return (size_t)tbik::rmsnorm_bwd_ws_floats(rows, H, dp, want_dw != 0) * sizeof(float);
}

int tbik_rmsnorm_backward(const tbik_bf16 *x, const tbik_bf16 *r, const tbik_bf16 *w,
                          const tbik_bf16 *dy, const tbik_bf16 *dr, tbik_bf16 *dh, float *dw,
                          int rows, int H, int64_t ld, float eps, int dp, float *ws,
                          size_t ws_bytes, void *stream) {
  if (!x || !r || !w || !dy || !dh) return TBIK_ERR_NULL;
  if (rows < 0 || H < 1 || H > 65536 || ld < H) return TBIK_ERR_SHAPE;
  if (!(eps >= 0.0f) || isinf(eps)) return TBIK_ERR_ARG;
  if (dw) {
    if (rows == 0 || (rows % 64) != 0) return TBIK_ERR_SHAPE;
    if (!tp_ok(dp) || (tbik::tree_T(rows / 64) % dp) != 0) return TBIK_ERR_TP;
    if ((rows / 64) / tbik::tree_T(rows / 64) > (1 << 20)) return TBIK_ERR_SHAPE;
  }
  if (!aligned(x, 2) || !aligned(r, 2) || !aligned(w, 2) || !aligned(dy, 2) || !aligned(dh, 2) ||
      (dr && !aligned(dr, 2)) || (dw && !aligned(dw, 4)))
    return TBIK_ERR_ALIGN;
  if (rows == 0) return TBIK_OK;
  if (!ws) return TBIK_ERR_WORKSPACE;
  if (!aligned(ws, 4)) return TBIK_ERR_ALIGN;
  if (ws_bytes < tbik_rmsnorm_backward_workspace_bytes(rows, H, dw ? dp : 1, dw != nullptr))
    return TBIK_ERR_WORKSPACE;
  return tbik::launch_rmsnorm_backward(x, r, w, dy, dr, dh, dw, rows, H, ld, eps, dw ? dp : 1, ws,
                                       as_stream(stream));
}

size_t tbik_logsoftmax_workspace_bytes(int M, int V, int tp) {
  (void)V;
  if (M < 0 || tp < 1) return 0;
  return (size_t)M * (size_t)tp * sizeof(float);
}

int tbik_logsoftmax_gather(const float *logits, int64_t ld, const int32_t *targets, float *out_lp,
                           int M, int V, int tp, float *ws, size_t ws_bytes, void *stream) {
  if (!logits || !targets || !out_lp) return TBIK_ERR_NULL;
  if (M < 0 || V < 1 || ld < V) return TBIK_ERR_SHAPE;
  if (!tp_ok(tp) || (tbik::tree_T(V) % tp) != 0) return TBIK_ERR_TP;
  if (!aligned(logits, 4) || !aligned(targets, 4) || !aligned(out_lp, 4)) return TBIK_ERR_ALIGN;
  if (M == 0) return TBIK_OK;
  if (M > 65535) return TBIK_ERR_SHAPE;
  if (!ws || ws_bytes < tbik_logsoftmax_workspace_bytes(M, V, tp)) return TBIK_ERR_WORKSPACE;
  if ((uintptr_t)ws & 3u) return TBIK_ERR_ALIGN;
  return tbik::launch_logsoftmax(logits, ld, targets, out_lp, M, V, tp, ws, nullptr, 0, 0,
                                 as_stream(stream));
}

int tbik_logsoftmax_gather_pmax(const float *logits, int64_t ld, const int32_t *targets,
                                float *out_lp, int M, int V, int tp, const float *pmax,
                                int64_t ld_pmax, int npmax, float *ws, size_t ws_bytes,
                                void *stream) {
  if (!logits || !targets || !out_lp || !pmax) return TBIK_ERR_NULL;
  if (M < 0 || V < 1 || ld < V || npmax < 1 || ld_pmax < npmax) return TBIK_ERR_SHAPE;
  if (!tp_ok(tp) || (tbik::tree_T(V) % tp) != 0) return TBIK_ERR_TP;
  if (!aligned(logits, 4) || !aligned(targets, 4) || !aligned(out_lp, 4) || !aligned(pmax, 4))
    return TBIK_ERR_ALIGN;
  if (M == 0) return TBIK_OK;
  if (M > 65535) return TBIK_ERR_SHAPE;
  if (!ws || ws_bytes < tbik_logsoftmax_workspace_bytes(M, V, tp)) return TBIK_ERR_WORKSPACE;
  if ((uintptr_t)ws & 3u) return TBIK_ERR_ALIGN;
  return tbik::launch_logsoftmax(logits, ld, targets, out_lp, M, V, tp, ws, pmax, ld_pmax, npmax,
                                 as_stream(stream));
}

int tbik_gemm_logits(const tbik_bf16 *A, int64_t lda, const tbik_bf16 *W, int64_t ldw, float *C,
                     int64_t ldc, int M, int N, int K, float *pmax, int64_t ld_pmax,
                     void *stream) {
  int rc = check_gemm(A, lda, W, ldw, C, ldc, nullptr, M, N, K, TBIK_LEAF_MFMA);
  if (rc) return rc;
  if (!C || !pmax) return TBIK_ERR_NULL;
  if (ld_pmax < (N + 63) / 64) return TBIK_ERR_SHAPE;
  if (!aligned(pmax, 4)) return TBIK_ERR_ALIGN;
  if (M == 0 || N == 0) return TBIK_OK;
  GemmCall c{};
  c.A = A; c.lda = lda; c.strideA = 0;
  c.W = W; c.ldw = ldw; c.strideW = 0;
  c.C = C; c.Cb = nullptr; c.ldc = ldc; c.strideC = 0; c.part_stride = 0;
  c.M = M; c.N = N; c.K = K; c.batch = 1; c.parts = 1; c.leaf_mode = TBIK_LEAF_MFMA;
  c.pmax = pmax; c.ld_pmax = ld_pmax;
  return tbik::launch_gemm(c, as_stream(stream));
}

int tbik_attention_causal(const tbik_bf16 *Q, int64_t ldq, const tbik_bf16 *K, int64_t ldk,
                          const tbik_bf16 *Vt, int64_t ldvt, tbik_bf16 *O, int64_t ldo, int L,
                          int heads, int head_dim, int batch, float scale, void *stream) {
  if (!Q || !K || !Vt || !O) return TBIK_ERR_NULL;
  if (head_dim != 128 || heads < 1 || batch < 0 || (int64_t)heads * batch > 65535)
    return TBIK_ERR_SHAPE;
  if (L != 64 && L != 128 && L != 256 && L != 512) return TBIK_ERR_SHAPE;
  if (ldq < (int64_t)heads * head_dim || ldk < (int64_t)heads * head_dim ||
      ldo < (int64_t)heads * head_dim || ldvt < (int64_t)batch * L)
    return TBIK_ERR_SHAPE;
  if (!ld_ok(ldq) || !ld_ok(ldk) || !ld_ok(ldvt) || !ld_ok(ldo)) return TBIK_ERR_ALIGN;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(Vt) || !aligned(O, 2)) return TBIK_ERR_ALIGN;
  if (!isfinite(scale)) return TBIK_ERR_ARG;
  if (batch == 0) return TBIK_OK;
  return tbik::launch_attn_causal(Q, ldq, K, ldk, Vt, ldvt, O, ldo, L, heads, batch, scale,
                                  as_stream(stream));
}

int tbik_gather_rows(const tbik_bf16 *table, int64_t ld_table, int rows, const int32_t *idx,
                     int n, int cols, tbik_bf16 *out, int64_t ld_out, void *stream) {
  if (!table || !idx || !out) return TBIK_ERR_NULL;
  if (rows < 0 || n < 0 || cols < 0 || ld_table < cols || ld_out < cols) return TBIK_ERR_SHAPE;
  if (!aligned(table, 2) || !aligned(idx, 4) || !aligned(out, 2)) return TBIK_ERR_ALIGN;
  if (n == 0 || cols == 0) return TBIK_OK;
  return tbik::launch_gather_rows(table, ld_table, rows, idx, n, cols, out, ld_out,
                                  as_stream(stream));
}

int tbik_softmax_causal(const float *S, int64_t ld_s, int64_t stride_s, tbik_bf16 *P,
                        int64_t ld_p, int64_t stride_p, int Lq, int Lk, int batch, int offset,
                        float scale, void *stream) {
  if (!S || !P) return TBIK_ERR_NULL;
  if (Lq < 0 || Lk < 1 || Lk > 65536 || batch < 0 || batch > 65535 || offset < 0)
    return TBIK_ERR_SHAPE;
  if (ld_s < Lk || ld_p < Lk || stride_s < 0 || stride_p < 0) return TBIK_ERR_SHAPE;
  if (!aligned(S, 4) || !aligned(P, 2)) return TBIK_ERR_ALIGN;
  if (!isfinite(scale)) return TBIK_ERR_ARG;
  if (Lq == 0 || batch == 0) return TBIK_OK;
  return tbik::launch_softmax_causal(S, ld_s, stride_s, P, ld_p, stride_p, Lq, Lk, batch, offset,
                                     scale, as_stream(stream));
}

int tbik_primitive(int op, const float *x, float *y, int64_t n, void *stream) {
  if (!x || !y) return TBIK_ERR_NULL;
  if (op < TBIK_PRIM_EXP || op > TBIK_PRIM_SILU) return TBIK_ERR_ARG;
  if (n < 0) return TBIK_ERR_SHAPE;
  if (((uintptr_t)x & 3u) || ((uintptr_t)y & 3u)) return TBIK_ERR_ALIGN;
  if (n == 0) return TBIK_OK;
  return tbik::launch_primitive(op, x, y, n, as_stream(stream));
}

}  // extern "C"
