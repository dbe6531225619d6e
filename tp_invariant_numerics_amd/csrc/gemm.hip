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

// ---------------------------------------------------------------------------
// Large-tile kernel: LDS ring fed by direct global->LDS loads.
//
// A workgroup of WAVES_M x WAVES_N waves owns an MT x NT output tile
// (MT = 16*WM*WAVES_M, NT = 16*WN*WAVES_N) and the whole K range of its part.
// Each 64-wide K block of A and W ("stage", (MT+NT)*128 bytes) is fetched once
// per workgroup with global_load_lds_dwordx4 into a ring of S LDS slots, S-1
// stages ahead of the MFMAs.  Inside a slot, row r's eight 16-byte chunks
// are stored XOR-swizzled (chunk c at position c ^ (r & 7)), so both the
// copy (one 8-row, 1 KB segment per wave instruction) and the MFMA fragment
// reads are free of bank conflicts.  Synchronisation is a wave-local wait on
// the vector-memory counter for the slot's own loads plus one s_barrier per
// K block; no fence is needed because the loads write LDS directly.
//
// The tree is the same as in k_gemm_mfma.  Leaves are taken in unrolled
// blocks of U (U | G): inside a block every merge is resolved at compile time
// and the merge of leaf j-1 is issued after the MFMAs of leaf j (two leaf
// accumulators), letting the VALU adds overlap the matrix unit.
//
// Tiles are numbered so that each XCD (workgroups are dealt to the 8 XCDs
// round-robin) receives a contiguous range, walked in groups of GROUP_M row
// tiles so that concurrently running tiles share A and W in that XCD's L2.
// ---------------------------------------------------------------------------
struct TileMap {
  int tiles_m, tiles_n, parts, group_m;
};

__device__ __forceinline__ int xcd_logical(int bid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int x = bid & 7, j = bid >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
}

typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int WM, int WN, int WAVES_M, int WAVES_N, int S, int U, int GD, int TD>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
k_gemm_ring(GemmArgs p, TileMap tm) {
  constexpr int WAVES = WAVES_M * WAVES_N;
  constexpr int MT = 16 * WM * WAVES_M;
  constexpr int NT = 16 * WN * WAVES_N;
  constexpr int R = 4 * WM * WN;
  constexpr int SEGA = MT / 8, SEGB = NT / 8;      // 1 KB segments per stage
  constexpr int SEG = SEGA + SEGB;
  static_assert(SEG % WAVES == 0, "segments must split evenly over waves");
  constexpr int DPW = SEG / WAVES;                  // loads per wave per stage
  constexpr int SLOT = SEG * 64;                    // 16-byte units per slot
  __shared__ u32x4 ring[S * SLOT];

  // ---- tile of this workgroup
  const int nblocks = tm.tiles_m * tm.tiles_n * tm.parts;
  int id = xcd_logical(blockIdx.x, nblocks);
  const int per_part = tm.tiles_m * tm.tiles_n;
  const int part = id / per_part;
  id -= part * per_part;
  const int span = tm.group_m * tm.tiles_n;
  const int grp = id / span;
  const int first_m = grp * tm.group_m;
  const int gsz = min(tm.tiles_m - first_m, tm.group_m);
  const int tile_m = first_m + (id - grp * span) % gsz;
  const int tile_n = (id - grp * span) / gsz;
  const int m0 = tile_m * MT, n0 = tile_n * NT;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N, wn = wave - (wave / WAVES_N) * WAVES_N;
  const int G = p.G;
  const int gpp = p.gpp;
  const int nleaf = gpp * G;
  const int64_t kbase = (int64_t)part * gpp * G * 64;

  // ---- this lane's source for each of its wave's DPW segments
  const uint16_t *src[DPW];
  int dst[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int seg = wave + WAVES * i;
    const int rin = lane >> 3;                       // row inside the segment
    const int c = (lane & 7) ^ rin;                  // logical chunk at this position
    if (seg < SEGA) {
      int row = m0 + seg * 8 + rin;
      row = row < p.M ? row : p.M - 1;
      src[i] = p.A + (int64_t)row * p.lda + kbase + 8 * c;
    } else {
      int row = n0 + (seg - SEGA) * 8 + rin;
      row = row < p.N ? row : p.N - 1;
      src[i] = p.W + (int64_t)row * p.ldw + kbase + 8 * c;
    }
    dst[i] = seg * 64;                               // segment base (16-byte units)
  }
  // ---- fragment offsets inside a slot (16-byte units)
  int fa[WM][2], fb[WN][2];
#pragma unroll
  for (int b = 0; b < WM; ++b) {
    const int row = wm * 16 * WM + 16 * b + (lane & 15);
#pragma unroll
    for (int h = 0; h < 2; ++h) fa[b][h] = row * 8 + ((4 * h + (lane >> 4)) ^ (row & 7));
  }
#pragma unroll
  for (int b = 0; b < WN; ++b) {
    const int row = MT + wn * 16 * WN + 16 * b + (lane & 15);
#pragma unroll
    for (int h = 0; h < 2; ++h) fb[b][h] = row * 8 + ((4 * h + (lane >> 4)) ^ (row & 7));
  }

  // issue the loads of stage `st` (clamped to the last stage: the surplus
  // loads at the end refill a slot that is never read again)
  auto issue = [&](int st) {
    const int sc = st < nleaf ? st : nleaf - 1;
    const int slot = st % S;
#pragma unroll
    for (int i = 0; i < DPW; ++i)
      __builtin_amdgcn_global_load_lds((gptr_t)(src[i] + (int64_t)sc * 64),
                                       (lptr_t)(ring + slot * SLOT + dst[i]), 16, 0, 0);
  };
  auto mfma_leaf = [&](float (&acc)[R], int st) {
    const u32x4 *sl = ring + (st % S) * SLOT;
    u32x4 a[WM][2], b[WN][2];
#pragma unroll
    for (int i = 0; i < WM; ++i) { a[i][0] = sl[fa[i][0]]; a[i][1] = sl[fa[i][1]]; }
#pragma unroll
    for (int i = 0; i < WN; ++i) { b[i][0] = sl[fb[i][0]]; b[i][1] = sl[fb[i][1]]; }
    leaf_mfma<WM, WN>(acc, a, b);
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st);

  // Leaves are processed in blocks of U (U divides G, so the lowest log2(U)
  // levels of PAIR inside a group are perfect trees over exactly these
  // blocks).  Inside a block every merge is static and the merge of leaf
  // j-1 follows the MFMAs of leaf j; block sums go through the runtime
  // stack `s` (PAIR over the G/U blocks of a group), group sums through `top`.
  constexpr int LU = U >= 8 ? 3 : U >= 4 ? 2 : U >= 2 ? 1 : 0;
  float s[GD > 0 ? GD : 1][R];
  float top[TD > 0 ? TD : 1][R];
  float node[R];
  const int nblk = G / U;
  int l = 0;
  for (int gi = 0; gi < gpp; ++gi) {
    for (int cb = 0; cb < nblk; ++cb) {
      float acc[2][R];
      float q[LU > 0 ? LU : 1][R];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        wait_vmcnt<DPW * (S - 2)>();
        __builtin_amdgcn_s_barrier();
        issue(l + S - 1);
        mfma_leaf(acc[j & 1], l);
        if (j > 0) pair_push<R, LU>(q, acc[(j - 1) & 1], j - 1, U);
        ++l;
      }
      pair_push<R, LU>(q, acc[(U - 1) & 1], U - 1, U);
#pragma unroll
      for (int r = 0; r < R; ++r) node[r] = acc[(U - 1) & 1][r];
      if (pair_push<R, GD>(s, node, cb, nblk)) pair_push<R, TD>(top, node, gi, gpp);
    }
  }
  wait_vmcnt<0>();     // no load into LDS may outlive the workgroup

  float *Cp = p.C ? p.C + (int64_t)part * p.part_stride : nullptr;
  uint16_t *Cbp = p.Cb;
  const int orow = 4 * (lane >> 4);
#pragma unroll
  for (int bm = 0; bm < WM; ++bm) {
#pragma unroll
    for (int bn = 0; bn < WN; ++bn) {
      const int col = n0 + wn * 16 * WN + 16 * bn + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * 16 * WM + 16 * bm + orow + i;
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

template <int WM, int WN, int WAVES_M, int WAVES_N, int S, int U, int GD, int TD>
static int launch_ring_cfg(const GemmArgs &a, hipStream_t s) {
  constexpr int MT = 16 * WM * WAVES_M, NT = 16 * WN * WAVES_N;
  TileMap tm;
  tm.tiles_m = (a.M + MT - 1) / MT;
  tm.tiles_n = (a.N + NT - 1) / NT;
  tm.parts = a.parts;
  tm.group_m = 8;
  const int64_t nb = (int64_t)tm.tiles_m * tm.tiles_n * tm.parts;
  if (nb > 0x7fffffff) return TBIK_ERR_SHAPE;
  hipLaunchKernelGGL((k_gemm_ring<WM, WN, WAVES_M, WAVES_N, S, U, GD, TD>), dim3((unsigned)nb),
                     dim3(64 * WAVES_M * WAVES_N), 0, s, a, tm);
  return check_launch();
}

// 128 x 64 tiles: 4 waves of 32 x 64 stacked along M; 4-stage ring (96 KB).
template <int U, int GD>
static int launch_ring_u(const GemmArgs &a, hipStream_t s) {
  switch (a.gpp) {
    case 1: return launch_ring_cfg<2, 4, 4, 1, 4, U, GD, 0>(a, s);
    case 2: return launch_ring_cfg<2, 4, 4, 1, 4, U, GD, 1>(a, s);
    case 4: return launch_ring_cfg<2, 4, 4, 1, 4, U, GD, 2>(a, s);
    case 8: return launch_ring_cfg<2, 4, 4, 1, 4, U, GD, 3>(a, s);
  }
  return TBIK_ERR_ARG;
}

// Block size U: the largest of 8, 4, 1 dividing G.  Stack depth for the
// PAIR over the G/U blocks: bit length of G/U - 1.
static bool ring_supported(int G) {
  const int U = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : 1;
  return bit_length(G / U - 1) <= (U == 1 ? 5 : 3);
}

static int launch_ring(const GemmArgs &a, hipStream_t s) {
  const int G = a.G;
  if (G % 8 == 0) {
    const int need = bit_length(G / 8 - 1);
    if (need == 0) return launch_ring_u<8, 0>(a, s);
    if (need <= 3) return launch_ring_u<8, 3>(a, s);
  }
  if (G % 4 == 0) {
    const int need = bit_length(G / 4 - 1);
    if (need == 0) return launch_ring_u<4, 0>(a, s);
    if (need <= 3) return launch_ring_u<4, 3>(a, s);
  }
  const int need = bit_length(G - 1);
  if (need <= 3) return launch_ring_u<1, 3>(a, s);
  if (need <= 5) return launch_ring_u<1, 5>(a, s);
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
  if (c.M > 32 && c.batch == 1 && ring_supported(a.G)) return launch_ring(a, s);
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
