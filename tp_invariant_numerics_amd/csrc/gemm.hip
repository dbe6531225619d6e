// gemm.hip -- tree-based invariant GEMM for gfx950.
//
// C[i,j] = TREE over K/64 leaves, leaf b = sum of A[i,k] W[j,k] over the
// 64-wide K block b (TBIK summary page, Abstract: TP-invariant matrix
// multiplication; IsoExec brief, section 叁: fixed accumulation blocking).
//
// MFMA leaf: two chained v_mfma_f32_16x16x32_bf16 from a zero accumulator.
// Lane l of a 64-wide wave holds, for both operands, the 8 consecutive k
// values 32h + 8(l/16) .. +7 of row (l mod 16) of its 16-row block, h being
// the index of the MFMA in the leaf.  The accumulator lane l, register i is
// output (4(l/16) + i, l mod 16) of the 16x16 block.  This instruction and
// operand mapping are the same in every kernel configuration below, so a
// leaf's bits depend only on its 64 A values and 64 W values.
//
// Tree: each wave streams its leaves through a register-tile binary-counter
// stack (tbik::pair_push) -- PAIR inside a group, then a second stack over
// the group sums.  Several waves of one workgroup may own disjoint, aligned
// group ranges of the same output tile; their nodes are combined through
// LDS by the perfect top of the tree.  A launch may also split K into
// `parts` aligned nodes written to a workspace (simulated tensor
// parallelism, TBIK "technical framework"); k_tree_combine finishes the tree.
// No atomics; no data-dependent reduction order.
#include "tbik_device.h"
#include "tbik_internal.h"
#include "../../include/tbik.h"

namespace tbik {

struct GemmArgs {
  const uint16_t *A; int64_t lda; int64_t strideA;
  const uint16_t *W; int64_t ldw; int64_t strideW;
  float *C; uint16_t *Cb; int64_t ldc; int64_t strideC; int64_t part_stride;
  int M, N;
  int G;        // leaves per group
  int gpp;      // groups per part
  int parts;
};

// Load one leaf's operand fragments for WB 16-row blocks (two MFMA halves).
template <int WB>
__device__ __forceinline__ void load_frags(u32x4 (&f)[WB][2], const uint16_t *const (&ptr)[WB],
                                           const bool (&valid)[WB], int64_t koff) {
#pragma unroll
  for (int b = 0; b < WB; ++b) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 v = *reinterpret_cast<const u32x4 *>(ptr[b] + koff + 32 * h);
      f[b][h] = valid[b] ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// One leaf for a WM x WN grid of 16x16 blocks: two chained MFMAs from zero.
template <int WM, int WN>
__device__ __forceinline__ void leaf_mfma(float (&out)[4 * WM * WN], const u32x4 (&fa)[WM][2],
                                          const u32x4 (&fb)[WN][2]) {
#pragma unroll
  for (int bm = 0; bm < WM; ++bm) {
#pragma unroll
    for (int bn = 0; bn < WN; ++bn) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[bm][0]),
                                                    __builtin_bit_cast(bf16x8, fb[bn][0]), acc,
                                                    0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[bm][1]),
                                                    __builtin_bit_cast(bf16x8, fb[bn][1]), acc,
                                                    0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) out[(bm * WN + bn) * 4 + i] = acc[i];
    }
  }
}

// WM x WN blocks of 16x16 per wave; WAVES waves side by side along N;
// KSPLIT wave groups own disjoint aligned group ranges of the same tile.
// GD: stack depth for PAIR inside a group (>= bit length of G-1).
// TD: stack depth over the groups of one wave group (log2 of their count).
template <int WM, int WN, int WAVES, int KSPLIT, int GD, int TD>
__global__ void __launch_bounds__(64 * WAVES * KSPLIT)
k_gemm_mfma(GemmArgs p) {
  constexpr int R = 4 * WM * WN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ks = wave / WAVES;
  const int wn = wave - ks * WAVES;
  const int part = blockIdx.z % p.parts;
  const int bat = blockIdx.z / p.parts;
  const int m0 = blockIdx.y * (16 * WM);
  const int n0 = (blockIdx.x * WAVES + wn) * (16 * WN);
  const int G = p.G;
  const int gpw = p.gpp / KSPLIT;               // groups of this wave group
  const int gfirst = part * p.gpp + ks * gpw;

  const uint16_t *A = p.A + (int64_t)bat * p.strideA;
  const uint16_t *W = p.W + (int64_t)bat * p.strideW;
  const int lr = lane & 15;
  const int lk = (lane >> 4) * 8;

  const uint16_t *ap[WM];
  bool av[WM];
#pragma unroll
  for (int b = 0; b < WM; ++b) {
    const int row = m0 + 16 * b + lr;
    av[b] = row < p.M;
    ap[b] = A + (int64_t)(av[b] ? row : 0) * p.lda + lk;
  }
  const uint16_t *wp[WN];
  bool wv[WN];
#pragma unroll
  for (int b = 0; b < WN; ++b) {
    const int col = n0 + 16 * b + lr;
    wv[b] = col < p.N;
    wp[b] = W + (int64_t)(wv[b] ? col : 0) * p.ldw + lk;
  }

  float s[GD > 0 ? GD : 1][R];
  float top[TD > 0 ? TD : 1][R];
  float node[R];

  const int nleaf = gpw * G;
  int64_t koff = (int64_t)gfirst * G * 64;
  u32x4 fa[WM][2], fb[WN][2];
  load_frags<WM>(fa, ap, av, koff);
  load_frags<WN>(fb, wp, wv, koff);
  int c = 0, gi = 0;
  for (int l = 0; l < nleaf; ++l) {
    u32x4 na[WM][2], nb[WN][2];
    const bool more = (l + 1) < nleaf;
    if (more) {
      load_frags<WM>(na, ap, av, koff + 64);
      load_frags<WN>(nb, wp, wv, koff + 64);
    }
    leaf_mfma<WM, WN>(node, fa, fb);
    if (pair_push<R, GD>(s, node, c, G)) {
      pair_push<R, TD>(top, node, gi, gpw);
      ++gi;
      c = 0;
    } else {
      ++c;
    }
    if (more) {
#pragma unroll
      for (int b = 0; b < WM; ++b) { fa[b][0] = na[b][0]; fa[b][1] = na[b][1]; }
#pragma unroll
      for (int b = 0; b < WN; ++b) { fb[b][0] = nb[b][0]; fb[b][1] = nb[b][1]; }
    }
    koff += 64;
  }
  // node = this wave group's node of the tree.

  if constexpr (KSPLIT > 1) {
    __shared__ float red[KSPLIT][WAVES][R][64];
#pragma unroll
    for (int r = 0; r < R; ++r) red[ks][wn][r][lane] = node[r];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v[KSPLIT];
#pragma unroll
      for (int q = 0; q < KSPLIT; ++q) v[q] = red[q][wn][r][lane];
#pragma unroll
      for (int w = KSPLIT; w > 1; w >>= 1) {
#pragma unroll
        for (int q = 0; q < w / 2; ++q) v[q] = v[2 * q] + v[2 * q + 1];
      }
      node[r] = v[0];
    }
  }

  float *Cp = p.C ? p.C + (int64_t)bat * p.strideC + (int64_t)part * p.part_stride : nullptr;
  uint16_t *Cbp = p.Cb ? p.Cb + (int64_t)bat * p.strideC : nullptr;
  const int orow = 4 * (lane >> 4);
#pragma unroll
  for (int bm = 0; bm < WM; ++bm) {
#pragma unroll
    for (int bn = 0; bn < WN; ++bn) {
      const int col = n0 + 16 * bn + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + 16 * bm + orow + i;
        if (row < p.M && col < p.N) {
          const float v = node[(bm * WN + bn) * 4 + i];
          const int64_t o = (int64_t)row * p.ldc + col;
          if (Cp) Cp[o] = v;
          if (Cbp) Cbp[o] = f2bf(v);
        }
      }
    }
  }
}

// Scalar leaves: one thread per output, 64 sequential fma per leaf in
// increasing k; the same tree.  Bit-exact with the CPU oracle.
__global__ void __launch_bounds__(64) k_gemm_scalar(GemmArgs p) {
  const int col = blockIdx.x * 64 + threadIdx.x;
  const int row = blockIdx.y;
  const int part = blockIdx.z % p.parts;
  const int bat = blockIdx.z / p.parts;
  if (col >= p.N) return;
  const uint16_t *a = p.A + (int64_t)bat * p.strideA + (int64_t)row * p.lda;
  const uint16_t *w = p.W + (int64_t)bat * p.strideW + (int64_t)col * p.ldw;
  const int G = p.G;
  float s[10][1];
  float top[3][1];
  float node[1];
  for (int gi = 0; gi < p.gpp; ++gi) {
    const int g = part * p.gpp + gi;
    for (int c = 0; c < G; ++c) {
      const int64_t kb = ((int64_t)g * G + c) * 64;
      float acc = 0.0f;
      for (int k = 0; k < 64; ++k) acc = __builtin_fmaf(bf2f(a[kb + k]), bf2f(w[kb + k]), acc);
      node[0] = acc;
      if (pair_push<1, 10>(s, node, c, G)) pair_push<1, 3>(top, node, gi, p.gpp);
    }
  }
  const int64_t o = (int64_t)row * p.ldc + col;
  if (p.C) p.C[(int64_t)bat * p.strideC + (int64_t)part * p.part_stride + o] = node[0];
  if (p.Cb) p.Cb[(int64_t)bat * p.strideC + o] = f2bf(node[0]);
}

// Top of the tree over tp dense [M,N] partials: a perfect binary tree.
template <int TP>
__device__ __forceinline__ float combine_tp(const float *ws, int64_t mn, int64_t idx) {
  float v[TP];
#pragma unroll
  for (int t = 0; t < TP; ++t) v[t] = ws[(int64_t)t * mn + idx];
#pragma unroll
  for (int w = TP; w > 1; w >>= 1) {
#pragma unroll
    for (int q = 0; q < w / 2; ++q) v[q] = v[2 * q] + v[2 * q + 1];
  }
  return v[0];
}

template <int TP>
__global__ void __launch_bounds__(256)
k_tree_combine(const float *ws, int64_t mn, int N, float *C, uint16_t *Cb, int64_t ldc) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < mn; idx += stride) {
    const float v = combine_tp<TP>(ws, mn, idx);
    const int64_t row = idx / N, col = idx - row * N;
    if (C) C[row * ldc + col] = v;
    if (Cb) Cb[row * ldc + col] = f2bf(v);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static int check_launch() {
  return hipGetLastError() == hipSuccess ? TBIK_OK : TBIK_ERR_LAUNCH;
}

template <int WM, int WN, int WAVES, int KSPLIT, int GD, int TD>
static int launch_cfg(const GemmArgs &a, int batch, hipStream_t s) {
  dim3 grid((unsigned)((a.N + 16 * WN * WAVES - 1) / (16 * WN * WAVES)),
            (unsigned)((a.M + 16 * WM - 1) / (16 * WM)), (unsigned)(batch * a.parts));
  hipLaunchKernelGGL((k_gemm_mfma<WM, WN, WAVES, KSPLIT, GD, TD>), grid, dim3(64 * WAVES * KSPLIT),
                     0, s, a);
  return check_launch();
}

// Large tiles: 32 x 16*WN per wave, 4 waves along N, one wave group per
// tile.  WN shrinks with the stack depth so the whole stack stays in
// registers.
template <int WN, int GD>
static int launch_big(const GemmArgs &a, int batch, hipStream_t s) {
  switch (a.gpp) {
    case 1: return launch_cfg<2, WN, 4, 1, GD, 0>(a, batch, s);
    case 2: return launch_cfg<2, WN, 4, 1, GD, 1>(a, batch, s);
    case 4: return launch_cfg<2, WN, 4, 1, GD, 2>(a, batch, s);
    case 8: return launch_cfg<2, WN, 4, 1, GD, 3>(a, batch, s);
  }
  return TBIK_ERR_ARG;
}

// Small M: one wave per group of the part, combined in LDS.
template <int WM, int GD>
static int launch_small(const GemmArgs &a, int batch, hipStream_t s) {
  switch (a.gpp) {
    case 1: return launch_cfg<WM, 1, 1, 1, GD, 0>(a, batch, s);
    case 2: return launch_cfg<WM, 1, 1, 2, GD, 0>(a, batch, s);
    case 4: return launch_cfg<WM, 1, 1, 4, GD, 0>(a, batch, s);
    case 8: return launch_cfg<WM, 1, 1, 8, GD, 0>(a, batch, s);
  }
  return TBIK_ERR_ARG;
}

int launch_gemm(const GemmCall &c, hipStream_t s) {
  const int nb = c.shard_of > 0 ? c.tree_leaves : c.K / 64;
  const int T = tree_T(nb);
  GemmArgs a;
  a.A = c.A; a.lda = c.lda; a.strideA = c.strideA;
  a.W = c.W; a.ldw = c.ldw; a.strideW = c.strideW;
  a.C = c.C; a.Cb = c.Cb; a.ldc = c.ldc; a.strideC = c.strideC; a.part_stride = c.part_stride;
  a.M = c.M; a.N = c.N;
  a.G = nb / T;
  a.parts = c.parts;
  a.gpp = T / (c.shard_of > 0 ? c.shard_of : c.parts);
  if (a.G > kMaxGroupLeaves) return TBIK_ERR_SHAPE;
  if ((int64_t)c.batch * c.parts > 65535) return TBIK_ERR_SHAPE;
  if (c.leaf_mode == TBIK_LEAF_SCALAR && c.M > 65535) return TBIK_ERR_SHAPE;
  if ((c.M + 15) / 16 > 65535) return TBIK_ERR_SHAPE;
  if (c.leaf_mode == TBIK_LEAF_SCALAR) {
    dim3 grid((unsigned)((c.N + 63) / 64), (unsigned)c.M, (unsigned)(c.batch * c.parts));
    hipLaunchKernelGGL(k_gemm_scalar, grid, dim3(64), 0, s, a);
    return check_launch();
  }
  const int need = bit_length(a.G - 1);
  if (c.M > 32 && need <= 5) {
    return need <= 3 ? launch_big<4, 3>(a, c.batch, s) : launch_big<2, 5>(a, c.batch, s);
  }
  if (c.M <= 16) {
    if (need <= 3) return launch_small<1, 3>(a, c.batch, s);
    if (need <= 5) return launch_small<1, 5>(a, c.batch, s);
    return launch_small<1, 9>(a, c.batch, s);
  }
  if (need <= 3) return launch_small<2, 3>(a, c.batch, s);
  if (need <= 5) return launch_small<2, 5>(a, c.batch, s);
  return launch_small<2, 9>(a, c.batch, s);
}

int launch_tree_combine(const float *ws, int tp, float *C, int64_t ldc, uint16_t *Cb, int M,
                        int N, hipStream_t s) {
  const int64_t mn = (int64_t)M * N;
  int64_t blocks = (mn + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks), block(256);
  switch (tp) {
    case 1: hipLaunchKernelGGL(k_tree_combine<1>, grid, block, 0, s, ws, mn, N, C, Cb, ldc); break;
    case 2: hipLaunchKernelGGL(k_tree_combine<2>, grid, block, 0, s, ws, mn, N, C, Cb, ldc); break;
    case 4: hipLaunchKernelGGL(k_tree_combine<4>, grid, block, 0, s, ws, mn, N, C, Cb, ldc); break;
    case 8: hipLaunchKernelGGL(k_tree_combine<8>, grid, block, 0, s, ws, mn, N, C, Cb, ldc); break;
    default: return TBIK_ERR_TP;
  }
  return check_launch();
}

}  // namespace tbik
