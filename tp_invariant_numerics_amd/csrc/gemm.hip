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
#include <type_traits>

#include "tbik_device.h"
#include "tbik_internal.h"
#include "../../include/tbik.h"

// Minimum split of 28-leaf-group GEMMs when a workspace is given.
#ifndef TBIK_SPLIT28_MIN
#define TBIK_SPLIT28_MIN 2
#endif

// Small-M kernel (M <= 16): each group's tree split over two waves (2) or
// not (1).
#ifndef TBIK_SMALL_GSPLIT
#define TBIK_SMALL_GSPLIT 2
#endif
// Small-M kernel: leaves of operand loads in flight ahead of the MFMAs.
#ifndef TBIK_SMALL_PF
#define TBIK_SMALL_PF 2
#endif

// Workgroups at or above which the wide ring kernel pairs parts (one per
// CU fills the chip)
#ifndef TBIK_RING_PPW_MIN_WG
#define TBIK_RING_PPW_MIN_WG 256
#endif

// Wide ring tiles with one group per part: all parts of a tile in one
// workgroup (1 = on)
#ifndef TBIK_RING_ALL_PARTS
#define TBIK_RING_ALL_PARTS 1
#endif


// 32-row ring tiles for 16 < M <= 32 (1 = on)
#ifndef TBIK_THIN
#define TBIK_THIN 1
#endif
#ifndef TBIK_THIN_MINB
#define TBIK_THIN_MINB 2
#endif
#ifndef TBIK_THIN_MIN_M
#define TBIK_THIN_MIN_M 0
#endif

// Narrow ring geometry: RING_WM x RING_WN 16x16 blocks per wave, 4 waves
// stacked along M, RING_S stages.
#ifndef TBIK_RING_WM
#define TBIK_RING_WM 2
#endif
#ifndef TBIK_RING_WN
#define TBIK_RING_WN 4
#endif
#ifndef TBIK_RING_S
#define TBIK_RING_S 4
#endif
#ifndef TBIK_RING_WAVES_M
#define TBIK_RING_WAVES_M 4
#endif
#ifndef TBIK_RING_WAVES_N
#define TBIK_RING_WAVES_N 1
#endif
// fragment reads one leaf ahead of the MFMAs (narrow tiles)
#ifndef TBIK_RING_PIPE
#define TBIK_RING_PIPE 1
#endif
// leaf accumulators per wave: 3 lets a leaf's merge overlap the next leaf's
// MFMAs, 2 saves one register tile
#ifndef TBIK_RING_NX
#define TBIK_RING_NX 3
#endif
// cache-policy bits of the ring's loads of A and of W (2 = non-temporal);
// W through tiles of at most 32 rows is streamed exactly once (every row
// tile holds all of M), so those loads are non-temporal (M = 1: 25 -> 22 us;
// the 128-row tiles share W between row tiles and lose with it)
#ifndef TBIK_RING_AUX_A
#define TBIK_RING_AUX_A 0
#endif
#ifndef TBIK_RING_AUX_B
#define TBIK_RING_AUX_B 0
#endif
#ifndef TBIK_THIN_AUX_B
#define TBIK_THIN_AUX_B 2
#endif

namespace tbik {

struct GemmArgs {
  const uint16_t *A; int64_t lda; int64_t strideA;
  const uint16_t *W; int64_t ldw; int64_t strideW;
  float *C; uint16_t *Cb; int64_t ldc; int64_t strideC; int64_t part_stride;
  int M, N;
  int G;        // leaves per group
  int gpp;      // groups per part
  int parts;
  // Optional (ring kernel, parts == 1): per-row maxima of C over 64-column
  // blocks, pmax[row * ld_pmax + col / 64].
  float *pmax; int64_t ld_pmax;
  // Optional (ring kernel, parts == 1, no C): glu = 1 (or 2 with the
  // activation rounded to bf16 before the product) makes the output columns
  // an interleave of W's two halves, 16 gate columns (W rows j) then their 16
  // up columns (rows N/2 + j), and the epilogue writes
  // H[row][j] = bf16(silu(bf16(gate)) * bf16(up)) instead of C.
  uint16_t *H; int64_t ldh; int glu;
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
// PF: leaves whose operand loads are in flight ahead of the MFMAs.
template <int WM, int WN, int WAVES, int KSPLIT, int GD, int TD, int PF = 1, int GSPLIT = 1>
__global__ void __launch_bounds__(64 * WAVES * KSPLIT * GSPLIT)
k_gemm_mfma(GemmArgs p) {
  constexpr int R = 4 * WM * WN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wg = wave / WAVES;                  // (group-split index, k split index)
  const int ks = wg / GSPLIT;
  const int gsi = wg - ks * GSPLIT;
  const int wn = wave - wg * WAVES;
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

  // GSPLIT = 2 (one group per wave group): the group's PAIR is split at its
  // binary decomposition -- the perfect tree over the first H leaves (H the
  // largest power of two below G) and PAIR over the other G - H, whose sum
  // is PAIR over the group -- and the two halves run on two waves.
  int Gw = G, lfirst = 0;
  if constexpr (GSPLIT == 2) {
    int H = 1;
    while (2 * H < G) H *= 2;
    Gw = gsi == 0 ? H : G - H;
    lfirst = gsi == 0 ? 0 : H;
  }
  const int nleaf = gpw * Gw;
  int64_t koff = ((int64_t)gfirst * G + lfirst) * 64;
  // Slot q of fa / fb holds the leaf l with l % PF == q: the loop is unrolled
  // by PF so that slots are named statically and no in-flight register is
  // copied; leaf l+PF is requested into the slot right after leaf l's MFMAs.
  u32x4 fa[PF][WM][2], fb[PF][WN][2];
#pragma unroll
  for (int q = 0; q < PF; ++q) {
    if (q < nleaf) {
      load_frags<WM>(fa[q], ap, av, koff + 64 * q);
      load_frags<WN>(fb[q], wp, wv, koff + 64 * q);
    }
  }
  int c = 0, gi = 0;
  for (int l0 = 0; l0 < nleaf; l0 += PF) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int l = l0 + q;
      if (l < nleaf) {
        leaf_mfma<WM, WN>(node, fa[q], fb[q]);
        if (l + PF < nleaf) {
          load_frags<WM>(fa[q], ap, av, koff + 64 * (q + PF));
          load_frags<WN>(fb[q], wp, wv, koff + 64 * (q + PF));
        }
        if (pair_push<R, GD>(s, node, c, Gw)) {
          pair_push<R, TD>(top, node, gi, gpw);
          ++gi;
          c = 0;
        } else {
          ++c;
        }
      }
    }
    koff += 64 * PF;
  }
  // node = this wave group's node of the tree.

  if constexpr (KSPLIT * GSPLIT > 1) {
    __shared__ float red[KSPLIT * GSPLIT][WAVES][R][64];
#pragma unroll
    for (int r = 0; r < R; ++r) red[wg][wn][r][lane] = node[r];
    __syncthreads();
    if (wg != 0) return;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v[KSPLIT];
#pragma unroll
      for (int q = 0; q < KSPLIT; ++q)
        v[q] = GSPLIT == 2 ? red[2 * q][wn][r][lane] + red[2 * q + 1][wn][r][lane]
                           : red[q][wn][r][lane];
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

// Barrier for the LDS ring: this wave's LDS reads are complete
// (lgkmcnt(0)) before it arrives, and the memory clobber keeps the compiler
// from moving LDS reads of a slot past the barrier after which that slot is
// refilled.  Unlike __syncthreads() it does not wait for outstanding global
// loads, so the ring's prefetches stay in flight.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

// Static merge schedule of one block of U leaves (U in {2,4,8}), leaf j in
// accumulator X[j % 3].  merge_leaf<j>() runs after the MFMAs of leaf j+1
// were issued (for j < U-1), so its adds can overlap them; every add writes
// its final destination (pair level P1, quad level P2), so no copies are
// needed.  The value returned by the merge of leaf U-1 is the block's PAIR
// (a perfect tree over the U leaves).
template <int R, int NX>
struct BlockTree {
  float X[NX][R];
  float P1[R];
  float P2[R];
};

template <int U, int J, int R, int NX>
__device__ __forceinline__ void merge_leaf(BlockTree<R, NX> &t, float (&out)[R]) {
  static_assert(U == 2 || U == 4 || U == 8, "block size");
  if constexpr ((J & 1) == 0) {
    return;                                     // waits for its sibling leaf
  } else {
    float(&a)[R] = t.X[(J - 1) % NX];
    float(&b)[R] = t.X[J % NX];
    constexpr int pairs = (J + 1) / 2;          // pairs completed so far
    if constexpr (U == 2) {
#pragma unroll
      for (int r = 0; r < R; ++r) out[r] = a[r] + b[r];
    } else if constexpr (pairs & 1) {
#pragma unroll
      for (int r = 0; r < R; ++r) t.P1[r] = a[r] + b[r];
    } else {
      float q[R];
#pragma unroll
      for (int r = 0; r < R; ++r) q[r] = t.P1[r] + (a[r] + b[r]);
      if constexpr (U == 4) {
#pragma unroll
        for (int r = 0; r < R; ++r) out[r] = q[r];
      } else if constexpr ((pairs / 2) & 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) t.P2[r] = q[r];
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) out[r] = t.P2[r] + q[r];
      }
    }
  }
}

constexpr int cbit_length(int v) { return v > 0 ? 1 + cbit_length(v >> 1) : 0; }

// Everything one wave of k_gemm_ring needs to stream leaves through the ring
// and merge them, plus the compile-time schedules of the tree.
template <int WM, int WN, int WAVES_M, int WAVES_N, int S, int NX, bool PIPE>
struct Ring {
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int MT = 16 * WM * WAVES_M;
  static constexpr int NT = 16 * WN * WAVES_N;
  static constexpr int R = 4 * WM * WN;
  static constexpr int SEGA = MT / 8, SEGB = NT / 8;     // 1 KB segments per stage
  static constexpr int SEG = SEGA + SEGB;
  static_assert(SEGA % WAVES == 0 && SEGB % WAVES == 0, "segments must split evenly");
  static constexpr int DPW = SEG / WAVES;                 // loads per wave per stage
  static constexpr int DPA = SEGA / WAVES;                // of which from A
  static constexpr int SLOT = SEG * 64;                   // 16-byte units per slot
  // Where a leaf issues the copy of the stage that refills the freed slot.
  // On tiles of 64 rows or more the copies go after the leaf's MFMAs: when
  // the memory pipeline is backed up a wave stalls at the load instruction,
  // and issued before the MFMAs that stall held back the matrix core (the
  // LM-head and prefill GEMMs ran 6% faster with the copies last, bitwise
  // the same).  The thin tiles keep them first (3% faster there).
  static constexpr bool LATE = MT >= 64;
  // store instructions per lane of a part's node on the multi-part path
  static constexpr int XSTORE = R;

  u32x4 *ring;
  __amdgpu_buffer_rsrc_t rsa, rsb;
  unsigned voff[DPW];
  int fa0[2], fb0[2];
  int wave, nleaf, l;
  int64_t kbase;

  // Copy stage `st` (this wave's share) into ring slot `slot`.  Past the
  // last leaf the loads still run, so that every wave's vector-memory count
  // advances by DPW per stage as the fixed waits expect, but through a
  // resource of zero size: out of range, they read no memory.
  __amdgpu_buffer_rsrc_t rs0;
  __device__ __forceinline__ void issue(int st, int slot) {
    const bool live = st < nleaf;
    const int soff = live ? (int)((kbase + (int64_t)st * 64) * 2) : 0;
    const __amdgpu_buffer_rsrc_t ra = live ? rsa : rs0, rb = live ? rsb : rs0;
#pragma unroll
    for (int i = 0; i < DPA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lptr_t)(ring + slot * SLOT + (wave + WAVES * i) * 64), 16, voff[i], soff, 0,
          TBIK_RING_AUX_A);
#pragma unroll
    for (int i = DPA; i < DPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (lptr_t)(ring + slot * SLOT + (wave + WAVES * i) * 64), 16, voff[i], soff, 0,
          MT <= 32 ? TBIK_THIN_AUX_B : TBIK_RING_AUX_B);
  }

  // fragments of the next leaf (PIPE): read one leaf ahead of their MFMAs
  u32x4 ca[WM][2], cb[WN][2];

  __device__ __forceinline__ void read_frags(u32x4 (&a)[WM][2], u32x4 (&b)[WN][2], int slot) {
    const u32x4 *sl = ring + slot * SLOT;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      a[i][0] = sl[fa0[0] + 128 * i];
      a[i][1] = sl[fa0[1] + 128 * i];
    }
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      b[i][0] = sl[fb0[0] + 128 * i];
      b[i][1] = sl[fb0[1] + 128 * i];
    }
  }

  __device__ __forceinline__ void mfma_leaf(float (&acc)[R], int slot) {
    u32x4 a[WM][2], b[WN][2];
    read_frags(a, b, slot);
    leaf_mfma<WM, WN>(acc, a, b);
  }

  // Prologue: the first S stages in flight (PIPE) or S-1 (otherwise); with
  // PIPE, also the first leaf's fragments.
  __device__ __forceinline__ void prologue() {
#pragma unroll
    for (int st = 0; st < (PIPE ? S : S - 1); ++st) issue(st, st);
    if constexpr (PIPE) {
      wait_vmcnt<DPW * (S - 1)>();
      ring_barrier();
      read_frags(ca, cb, 0);
    }
  }

  // One leaf: wait for its stage, the MFMAs, and the refill of the slot the
  // previous leaf freed (before or after the MFMAs, see LATE).
  // `static_slot`: the slot is known at compile time (the block started at a
  // multiple of S).
  // XS: store instructions this wave issued after the loads of the stages
  // still in flight (a previous part's node, see k_gemm_ring): the first
  // S - 1 leaves of the next part allow them in the wait, since the
  // vector-memory counter retires loads and stores in issue order.
  template <int XS = 0>
  __device__ __forceinline__ void step(float (&acc)[R], int j, bool static_slot) {
    // keep the scheduler inside one leaf: unbounded interleaving across a
    // fully unrolled group raises register pressure into spills
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<DPW * (S - 2) + XS>();
    ring_barrier();
    if constexpr (PIPE) {
      // stage l+j+1 has landed; leaf l+j's slot is free (its fragments are
      // in ca/cb): refill it with stage l+j+S, read the next leaf's
      // fragments, then the MFMAs of leaf l+j
      u32x4 na[WM][2], nb[WN][2];
      if constexpr (!LATE) {
        if (static_slot) issue(l + j + S, j % S);
        else issue(l + j + S, (unsigned)(l + j) % S);
      }
      if (static_slot) read_frags(na, nb, (j + 1) % S);
      else read_frags(na, nb, (unsigned)(l + j + 1) % S);
      leaf_mfma<WM, WN>(acc, ca, cb);
      if constexpr (LATE) {
        __builtin_amdgcn_sched_barrier(0);
        if (static_slot) issue(l + j + S, j % S);
        else issue(l + j + S, (unsigned)(l + j) % S);
      }
#pragma unroll
      for (int i = 0; i < WM; ++i) { ca[i][0] = na[i][0]; ca[i][1] = na[i][1]; }
#pragma unroll
      for (int i = 0; i < WN; ++i) { cb[i][0] = nb[i][0]; cb[i][1] = nb[i][1]; }
    } else if (static_slot) {
      if constexpr (!LATE) issue(l + j + S - 1, (j + S - 1) % S);
      mfma_leaf(acc, j % S);
      if constexpr (LATE) {
        __builtin_amdgcn_sched_barrier(0);
        issue(l + j + S - 1, (j + S - 1) % S);
      }
    } else {
      if constexpr (!LATE) issue(l + j + S - 1, (unsigned)(l + j + S - 1) % S);
      mfma_leaf(acc, (unsigned)(l + j) % S);
      if constexpr (LATE) {
        __builtin_amdgcn_sched_barrier(0);
        issue(l + j + S - 1, (unsigned)(l + j + S - 1) % S);
      }
    }
  }


  // Perfect tree over the next U leaves (U in {1,2,4,8}), merges resolved at
  // compile time; with NX == 3 the merge of leaf j-1 follows the MFMAs of
  // leaf j.  Advances l by U.
  // AL: the block is known to start at a leaf index that is a multiple of
  // U (then, with U % S == 0, its ring slots are known at compile time).
  // XWN: this subtree's leading leaves that take the extra wait of XSTORE
  // stores (at most S - 1, the first leaves of a part after a part's node
  // went out).
  template <int U, bool AL = true, int XWN = 0>
  __device__ __forceinline__ void block(float (&out)[R]) {
    if constexpr (U == 1) {
      step<(XWN > 0 ? XSTORE : 0)>(out, 0, false);
      l += 1;
    } else {
      constexpr bool SS = AL && (U % S) == 0;
      BlockTree<R, NX> bt;
#define TBIK_LEAF_STEP(J)                                                    \
  if constexpr ((J) < U) {                                                   \
    if constexpr (NX == 2 && (J) > 0) merge_leaf<U, (J) - 1, R, NX>(bt, out); \
    step<((J) < XWN ? XSTORE : 0)>(bt.X[(J) % NX], (J), SS);                \
    if constexpr (NX == 3 && (J) > 0) merge_leaf<U, (J) - 1, R, NX>(bt, out); \
  }
      TBIK_LEAF_STEP(0) TBIK_LEAF_STEP(1) TBIK_LEAF_STEP(2) TBIK_LEAF_STEP(3)
      TBIK_LEAF_STEP(4) TBIK_LEAF_STEP(5) TBIK_LEAF_STEP(6) TBIK_LEAF_STEP(7)
#undef TBIK_LEAF_STEP
      merge_leaf<U, U - 1, R, NX>(bt, out);
      l += U;
    }
  }

  // Perfect tree over N leaves (N a power of two): halves recursively,
  // blocks of at most 8 leaves at the bottom.
  template <int N, bool AL = true, int XWN = 0>
  __device__ __forceinline__ void perfect(float (&out)[R]) {
    if constexpr (N <= 8) {
      block<N, AL, XWN>(out);
    } else {
      float left[R];
      perfect<N / 2, AL, XWN>(left);
      perfect<N / 2, AL, (XWN > N / 2 ? XWN - N / 2 : 0)>(out);
#pragma unroll
      for (int r = 0; r < R; ++r) out[r] = left[r] + out[r];
    }
  }

  // PAIR over N leaves: the perfect tree over the largest power-of-two
  // prefix, added to PAIR over the rest (an odd tail moves up unchanged, so
  // PAIR is this right fold of its binary decomposition).
  template <int N, bool AL = true, int XWN = 0>
  __device__ __forceinline__ void pair(float (&out)[R]) {
    constexpr int H = (N >= 256) ? 256 : (N >= 128) ? 128 : (N >= 64) ? 64 : (N >= 32) ? 32
                    : (N >= 16) ? 16 : (N >= 8) ? 8 : (N >= 4) ? 4 : (N >= 2) ? 2 : 1;
    if constexpr (H == N) {
      perfect<N, AL, XWN>(out);
    } else {
      float left[R];
      perfect<H, AL, XWN>(left);
      pair<N - H, AL, (XWN > H ? XWN - H : 0)>(out);
#pragma unroll
      for (int r = 0; r < R; ++r) out[r] = left[r] + out[r];
    }
  }
};

// GS > 0: the group size G is the compile-time constant GS; U == 0 then
// evaluates each group as one Ring::pair<GS>, any other U as 8-leaf blocks
// plus a static tail.  GS == 0: runtime G, blocks of U leaves
// pushed through a binary-counter stack of depth GD.  TD: stack depth over
// the groups of one part.
//
// PPW: consecutive parts (K ranges) per workgroup.  With PPW > 1 a workgroup
// streams its parts' leaves through one continuous ring and writes each
// part's node to that part's slot as soon as the part is done, so the next
// part's first stages are already in flight; each part's tree is unchanged.
template <int WM, int WN, int WAVES_M, int WAVES_N, int S, int NX, bool PIPE, int GS, int U, int GD,
          int TD, int MINB, int PPW = 1>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, MINB)
k_gemm_ring(GemmArgs p, TileMap tm) {
  // The body uses buffer-resource builtins that only exist for the device;
  // the host compilation pass only needs the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  using RG = Ring<WM, WN, WAVES_M, WAVES_N, S, NX, PIPE>;
  static_assert(PPW == 1 || (RG::LATE && !PIPE),
                "several parts per workgroup: S - 1 stages in flight at a part's end");
  constexpr int MT = RG::MT, NT = RG::NT, R = RG::R, WAVES = RG::WAVES;
  constexpr int DPW = RG::DPW, DPA = RG::DPA, SEGA = RG::SEGA;
  __shared__ u32x4 ring[S * RG::SLOT];

  // ---- tile of this workgroup
  const int nblocks = tm.tiles_m * tm.tiles_n * (tm.parts / PPW);
  int id = xcd_logical(blockIdx.x, nblocks);
  const int per_part = tm.tiles_m * tm.tiles_n;
  const int part0 = (id / per_part) * PPW;          // first of this workgroup's parts
  id -= (id / per_part) * per_part;
  const int span = tm.group_m * tm.tiles_n;
  const int grp = id / span;
  const int first_m = grp * tm.group_m;
  const int gsz = min(tm.tiles_m - first_m, tm.group_m);
  const int tile_m = first_m + (id - grp * span) % gsz;
  const int tile_n = (id - grp * span) / gsz;
  const int m0 = tile_m * MT, n0 = tile_n * NT;

  const int lane = threadIdx.x & 63;
  RG rg;
  rg.ring = ring;
  rg.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = rg.wave;
  const int wm = wave / WAVES_N, wn = wave - (wave / WAVES_N) * WAVES_N;
  const int G = GS > 0 ? GS : p.G;
  const int gpp = p.gpp;
  rg.nleaf = PPW * gpp * G;
  rg.kbase = (int64_t)part0 * gpp * G * 64;
  rg.l = 0;

  // ---- buffer resources over this tile's rows (rows past the end are
  //      clamped to the last row, so every access stays inside)
  const int arows = min(MT, p.M - m0), brows = min(NT, p.N - n0);
  const bool glu = p.glu != 0;
  rg.rsa = __builtin_amdgcn_make_buffer_rsrc((void *)(p.A + (int64_t)m0 * p.lda), (short)0,
                                             (int)((int64_t)arows * p.lda * 2), 0x00020000);
  // SwiGLU mode: the tile's columns map to rows of both halves of W, so the
  // resource covers all of W
  rg.rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(glu ? p.W : p.W + (int64_t)n0 * p.ldw), (short)0,
      (int)((int64_t)(glu ? p.N : brows) * p.ldw * 2), 0x00020000);
  rg.rs0 = __builtin_amdgcn_make_buffer_rsrc((void *)p.W, (short)0, 0, 0x00020000);
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int seg = wave + WAVES * i;
    const int rin = lane >> 3;
    const int c = (lane & 7) ^ rin;                  // logical chunk at this position
    if (i < DPA) {
      const int row = min(seg * 8 + rin, arows - 1);
      rg.voff[i] = (unsigned)(((int64_t)row * p.lda + 8 * c) * 2);
    } else {
      int row = min((seg - SEGA) * 8 + rin, brows - 1);
      if (glu) {                                     // interleaved column -> row of W
        const int ic = n0 + row;
        row = ((ic & 31) < 16 ? 0 : p.N / 2) + (ic >> 5) * 16 + (ic & 15);
      }
      rg.voff[i] = (unsigned)(((int64_t)row * p.ldw + 8 * c) * 2);
    }
  }
  // ---- fragment bases (16-byte units) inside slot 0; the row's low three
  //      bits equal lane & 7, so the swizzle only depends on the lane
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    rg.fa0[h] = (wm * 16 * WM + lr) * 8 + ((4 * h + lg) ^ (lr & 7));
    rg.fb0[h] = (MT + wn * 16 * WN + lr) * 8 + ((4 * h + lg) ^ (lr & 7));
  }

  rg.prologue();

  float node[R];
  const int orow = 4 * (lane >> 4);
  bool staged = false;                  // the last part's output went out through LDS
  // The tree of one part.  Its first XWV leaves (the first leaves of its
  // first group) also allow the previous part's node stores in their waits
  // (several parts per workgroup, below).
#define TBIK_PART_TREE(XWV)                                                        \
  for (int gi = 0; gi < ngroups; ++gi) {                                           \
    if constexpr (GS > 0 && U == 0) {                                              \
      /* the whole group as one compile-time PAIR (perfect trees over the */      \
      /* binary decomposition of GS, right-folded): one node fewer live */        \
      /* than blocks of 8 pushed through a stack; same tree, same bits */         \
      if ((XWV) > 0 && gi == 0) rg.template pair<GS, (GS % S) == 0, (XWV)>(node);  \
      else rg.template pair<GS, (GS % S) == 0>(node);                              \
    } else if constexpr (GS > 0) {                                                 \
      /* full 8-leaf blocks (perfect subtrees, aligned in the group) in a */      \
      /* loop, then the static tail of GS % 8 leaves; PAIR over the group */      \
      /* is PAIR over these block values, the tail's PAIR the last item. */       \
      /* Ring slots are static only if every group starts at a multiple */       \
      /* of S leaves (GS % S == 0). */                                             \
      constexpr int NB = GS / 8, TAIL = GS % 8, NI = NB + (TAIL ? 1 : 0);          \
      constexpr int ID = cbit_length(NI - 1);                                      \
      constexpr bool AL = (GS % S) == 0;                                           \
      float st[ID > 0 ? ID : 1][R];                                                \
      _Pragma("clang loop unroll(disable)")                                        \
      for (int b = 0; b < NB; ++b) {                                               \
        if ((XWV) > 0 && gi == 0 && b == 0) rg.template block<8, AL, (XWV)>(node); \
        else rg.template block<8, AL>(node);                                       \
        pair_push<R, ID>(st, node, b, NI);                                         \
      }                                                                            \
      if constexpr (TAIL > 0) {                                                    \
        if (NB == 0 && (XWV) > 0 && gi == 0) rg.template pair<TAIL, AL, (XWV)>(node); \
        else rg.template pair<TAIL, AL>(node);                                     \
        pair_push<R, ID>(st, node, NB, NI);                                        \
      }                                                                            \
    } else {                                                                       \
      float s[GD > 0 ? GD : 1][R];                                                 \
      const int nblk = G / U;                                                      \
      for (int cb = 0; cb < nblk; ++cb) {                                          \
        rg.template block<U>(node);                                                \
        pair_push<R, GD>(s, node, cb, nblk);                                       \
      }                                                                            \
    }                                                                              \
    pair_push<R, TD>(top, node, gi, gpp);                                          \
  }

  if constexpr (PPW == 1) {
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
  const int part = part0 + pi;
  float top[TD > 0 ? TD : 1][R];
  const int ngroups = gpp;
  TBIK_PART_TREE(0)
  wait_vmcnt<0>();                        // no load into LDS may outlive the workgroup

  if (glu) {
    // a wave's 16 * WN columns start at a multiple of 32: block pairs
    // (2q, 2q+1) are the gate and up columns of the same 16 units, held by
    // the same lane; the arithmetic is the SwiGLU node's on the GEMM's bf16
    // outputs
#pragma unroll
    for (int bm = 0; bm < WM; ++bm) {
#pragma unroll
      for (int q = 0; q < WN / 2; ++q) {
        const int colg = n0 + wn * 16 * WN + 32 * q + (lane & 15);
        const int unit = (colg >> 5) * 16 + (colg & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m0 + wm * 16 * WM + 16 * bm + orow + i;
          if (row < p.M && colg < p.N) {
            float a = silu(bf_round(node[(bm * WN + 2 * q) * 4 + i]));
            if (p.glu == 2) a = bf_round(a);
            p.H[(int64_t)row * p.ldh + unit] = f2bf(a * bf_round(node[(bm * WN + 2 * q + 1) * 4 + i]));
          }
        }
      }
    }
    continue;
  }
  float *Cp = p.C ? p.C + (int64_t)part * p.part_stride : nullptr;
  uint16_t *Cbp = p.Cb;
  staged = false;
  // fp32 or bf16 output of a workgroup's only part: the tile goes through
  // LDS (the ring is free: every copy has landed, vmcnt 0 above) and out as
  // whole rows, 16 bytes per lane, non-temporal, so every store instruction
  // writes full lines (the MFMA layout alone gives 64-byte fp32 or 32-byte
  // bf16 row pieces).  With 128-column tiles the 64-column row maxima are
  // formed from the same LDS rows as they are stored (16 lanes hold one
  // row's 64 columns), with no separate phase.
  constexpr int LDO = NT + 4;                         // padded row (conflict-free writes)
  constexpr int LPR = NT / 4;                         // lanes per tile row
  constexpr int RPI = 64 / LPR;                       // rows per store instruction
  constexpr int RPW = MT / WAVES;                     // rows per wave
  if constexpr (PPW == 1 && MT >= 64 && RPW % RPI == 0 &&
                MT * LDO * 4 <= S * RG::SLOT * 16) {
    if (Cp && !Cbp && (p.ldc & 3) == 0 && ((uintptr_t)Cp & 15) == 0) {
      staged = true;
      float *st = reinterpret_cast<float *>(ring);
      ring_barrier();                                 // every wave is past its last fragment read
#pragma unroll
      for (int bm = 0; bm < WM; ++bm)
#pragma unroll
        for (int bn = 0; bn < WN; ++bn)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            st[(wm * 16 * WM + 16 * bm + orow + i) * LDO + wn * 16 * WN + 16 * bn + (lane & 15)] =
                node[(bm * WN + bn) * 4 + i];
      ring_barrier();
      const int cl = 4 * (lane % LPR);
      const int col = n0 + cl;
#pragma unroll
      for (int r0 = 0; r0 < RPW; r0 += RPI) {
        const int rl = wave * RPW + r0 + lane / LPR;
        const f32x4 v = *reinterpret_cast<const f32x4 *>(st + rl * LDO + cl);
        const int row = m0 + rl;
        if (row < p.M) {
          float *dst = Cp + (int64_t)row * p.ldc + col;
          if (col + 3 < p.N) {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(dst));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < p.N) dst[e] = v[e];
          }
        }
        if constexpr (NT == 128) {
          if (p.pmax) {
            // lanes 16k .. 16k+15 hold one row's 64-column block; every lane
            // takes part in the DPP steps (a lane past M or N contributes
            // -inf), the block's last lane stores the maximum
            float mx = -__builtin_inff();
            if (row < p.M) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < p.N) mx = __builtin_fmaxf(mx, v[e]);
            }
            mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                         0x111, 0xf, 0xf, false)));
            mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                         0x112, 0xf, 0xf, false)));
            mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                         0x114, 0xf, 0xf, false)));
            mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                         0x118, 0xf, 0xf, false)));
            const int cb = n0 + 64 * ((lane >> 4) & 1);
            if ((lane & 15) == 15 && row < p.M && cb < p.N)
              p.pmax[(int64_t)row * p.ld_pmax + cb / 64] = mx;
          }
        }
      }
    } else if (!Cp && Cbp && (p.ldc & 7) == 0 && ((uintptr_t)Cbp & 15) == 0) {
      // bf16-only output (the decoder's projections): the same, rounded to
      // bf16 on the way into LDS, 8 values (16 bytes) per lane, non-temporal
      constexpr int LDB = NT + 8;                     // padded row, in bf16 elements
      constexpr int LPB = NT / 8;                     // lanes per tile row
      constexpr int RPB = 64 / LPB;                   // rows per store instruction
      static_assert(RPW % RPB == 0 && MT * LDB * 2 <= S * RG::SLOT * 16, "bf16 staging");
      staged = true;
      uint16_t *sb = reinterpret_cast<uint16_t *>(ring);
      ring_barrier();                                 // every wave is past its last fragment read
#pragma unroll
      for (int bm = 0; bm < WM; ++bm)
#pragma unroll
        for (int bn = 0; bn < WN; ++bn)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sb[(wm * 16 * WM + 16 * bm + orow + i) * LDB + wn * 16 * WN + 16 * bn + (lane & 15)] =
                f2bf(node[(bm * WN + bn) * 4 + i]);
      ring_barrier();
      const int cl = 8 * (lane % LPB);
      const int col = n0 + cl;
#pragma unroll
      for (int r0 = 0; r0 < RPW; r0 += RPB) {
        const int rl = wave * RPW + r0 + lane / LPB;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(sb + rl * LDB + cl);
        const int row = m0 + rl;
        if (row < p.M) {
          uint16_t *dst = Cbp + (int64_t)row * p.ldc + col;
          if (col + 7 < p.N) {
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
          } else {
            const uint16_t *e16 = sb + rl * LDB + cl;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (col + e < p.N) dst[e] = e16[e];
          }
        }
      }
    }
  }
  if (!staged) {
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
  }
  } else {
  // Several parts per workgroup: a part's node leaves as exactly RG::XSTORE
  // buffer stores per lane (an element outside C sent past the end of the
  // buffer range, no branch: fp32 only, which the launcher checks), issued
  // behind the S - 1 stages already in flight for the next part; that
  // part's first S - 1 leaves count them in their waits (TBIK_PART_TREE).
  // (The part's tree and its node inside one function: with the tree
  // outside it, the compiler spills the multi-part kernels heavily.)
  auto run_part = [&](auto xw_tag, const int pi) {
    constexpr int XW = decltype(xw_tag)::value;
    float top[TD > 0 ? TD : 1][R];
    const int ngroups = gpp;
    TBIK_PART_TREE(XW)
    if (pi == PPW - 1) wait_vmcnt<0>();   // no load into LDS may outlive the workgroup
    float *Cp = p.C + (int64_t)(part0 + pi) * p.part_stride;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(Cp + (int64_t)m0 * p.ldc), (short)0, (int)((int64_t)arows * p.ldc * 4),
        0x00020000);
#pragma unroll
    for (int bm = 0; bm < WM; ++bm) {
#pragma unroll
      for (int bn = 0; bn < WN; ++bn) {
        const int col = n0 + wn * 16 * WN + 16 * bn + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rl = wm * 16 * WM + 16 * bm + orow + i;
          const bool in = rl < arows && col < p.N;
          const unsigned off = in ? (unsigned)(((int64_t)rl * p.ldc + col) * 4) : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t,
                                                node[(bm * WN + bn) * 4 + i]), rc, off, 0, 0);
        }
      }
    }
  };
  run_part(std::integral_constant<int, 0>{}, 0);
  // the later parts, one per iteration (one copy of their tree)
#pragma clang loop unroll(disable)
  for (int pi = 1; pi < PPW; ++pi) run_part(std::integral_constant<int, S - 1>{}, pi);
  }
#undef TBIK_PART_TREE
  if constexpr (PPW > 1) {
    // no row maxima with several parts per workgroup (the launcher refuses)
  } else if constexpr (WN == 4) {
    // Exact row maxima of this wave's 64 columns (max is order-free): the
    // logprob path's log-softmax then reads the logits only once.
    if (p.pmax) {
      const int cblk = (n0 + wn * 16 * WN) / 64;
#pragma unroll
      for (int bm = 0; bm < WM; ++bm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float mx = -__builtin_inff();
#pragma unroll
          for (int bn = 0; bn < WN; ++bn) {
            const int col = n0 + wn * 16 * WN + 16 * bn + (lane & 15);
            if (col < p.N) mx = __builtin_fmaxf(mx, node[(bm * WN + bn) * 4 + i]);
          }
          // running maximum along each 16-lane row (DPP row_shr 1, 2, 4, 8;
          // a lane without a source keeps its own value): lane 15 of the
          // row ends with the maximum of all 16 lanes
          mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                       0x111, 0xf, 0xf, false)));
          mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                       0x112, 0xf, 0xf, false)));
          mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                       0x114, 0xf, 0xf, false)));
          mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                       0x118, 0xf, 0xf, false)));
          const int row = m0 + wm * 16 * WM + 16 * bm + orow + i;
          if ((lane & 15) == 15 && row < p.M && n0 + wn * 16 * WN < p.N)
            p.pmax[(int64_t)row * p.ld_pmax + cblk] = mx;
        }
      }
    }
  } else if constexpr (WN == 2 && WAVES_N == 4) {
    // 32-column waves, output not staged (the staged path forms the row
    // maxima as it stores): each wave's row maxima over its 32 columns go to
    // LDS (the ring is free once every wave is past its last leaf), then
    // the two halves of each 64-column block are combined.
    if (p.pmax && !staged) {
      float *pm = reinterpret_cast<float *>(ring);    // [MT rows][WAVES_N]
      // LDS-only barriers: every wave has drained its loads into the ring
      // (vmcnt 0 above); a full __syncthreads would also wait for the C
      // stores just issued
      ring_barrier();
#pragma unroll
      for (int bm = 0; bm < WM; ++bm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float mx = -__builtin_inff();
#pragma unroll
          for (int bn = 0; bn < WN; ++bn) {
            const int col = n0 + wn * 16 * WN + 16 * bn + (lane & 15);
            if (col < p.N) mx = __builtin_fmaxf(mx, node[(bm * WN + bn) * 4 + i]);
          }
          mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                       0x111, 0xf, 0xf, false)));
          mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                       0x112, 0xf, 0xf, false)));
          mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                       0x114, 0xf, 0xf, false)));
          mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       __builtin_bit_cast(int, mx), __builtin_bit_cast(int, mx),
                                       0x118, 0xf, 0xf, false)));
          if ((lane & 15) == 15) pm[(wm * 16 * WM + 16 * bm + orow + i) * WAVES_N + wn] = mx;
        }
      }
      ring_barrier();
      for (int e = threadIdx.x; e < MT * (WAVES_N / 2); e += 64 * WAVES) {
        const int r = e / (WAVES_N / 2), b = e - r * (WAVES_N / 2);
        const int row = m0 + r, c0 = n0 + 64 * b;
        if (row < p.M && c0 < p.N)
          p.pmax[(int64_t)row * p.ld_pmax + c0 / 64] =
              __builtin_fmaxf(pm[r * WAVES_N + 2 * b], pm[r * WAVES_N + 2 * b + 1]);
      }
    }
  }
#endif
}

static int check_launch() {
  return hipGetLastError() == hipSuccess ? TBIK_OK : TBIK_ERR_LAUNCH;
}

// Row maxima over 64-column blocks of an fp32 matrix (the fused epilogue's
// result for shapes the ring kernel does not take): one thread per block.
__global__ void __launch_bounds__(256)
k_block_rowmax(const float *C, int64_t ldc, int M, int N, float *pmax, int64_t ld_pmax) {
  const int nblk = (N + 63) / 64;
  const int64_t total = (int64_t)M * nblk;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = t / nblk;
    const int b = (int)(t - row * nblk);
    const float *c = C + row * ldc + (int64_t)b * 64;
    const int n = N - b * 64 < 64 ? N - b * 64 : 64;
    float mx = -__builtin_inff();
    for (int j = 0; j < n; ++j) mx = __builtin_fmaxf(mx, c[j]);
    pmax[row * ld_pmax + b] = mx;
  }
}

int launch_block_rowmax(const float *C, int64_t ldc, int M, int N, float *pmax, int64_t ld_pmax,
                        hipStream_t s) {
  const int64_t total = (int64_t)M * ((N + 63) / 64);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_block_rowmax, dim3((unsigned)blocks), dim3(256), 0, s, C, ldc, M, N, pmax,
                     ld_pmax);
  return check_launch();
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

// Four consecutive elements of a row per thread (N % 4 == 0, 16-byte
// aligned partials and fp32 output rows, 8-byte aligned bf16 rows).
template <int TP>
__global__ void __launch_bounds__(256)
k_tree_combine4(const float *ws, int64_t mn, int N, float *C, uint16_t *Cb, int64_t ldc) {
  const int64_t n4 = mn / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += stride) {
    f32x4 v[TP];
#pragma unroll
    for (int t = 0; t < TP; ++t)
      v[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(ws + (int64_t)t * mn + 4 * q));
#pragma unroll
    for (int w = TP; w > 1; w >>= 1) {
#pragma unroll
      for (int k = 0; k < w / 2; ++k) v[k] = v[2 * k] + v[2 * k + 1];
    }
    const int64_t idx = 4 * q;
    const int64_t row = idx / N, col = idx - row * N;
    if (C) __builtin_nontemporal_store(v[0], reinterpret_cast<f32x4 *>(C + row * ldc + col));
    if (Cb) {
      u32x2 o;
      o[0] = pack_bf16(v[0][0], v[0][1]);
      o[1] = pack_bf16(v[0][2], v[0][3]);
      *reinterpret_cast<u32x2 *>(Cb + row * ldc + col) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------


template <int WM, int WN, int WAVES, int KSPLIT, int GD, int TD, int PF = 1, int GSPLIT = 1>
static int launch_cfg(const GemmArgs &a, int batch, hipStream_t s) {
  dim3 grid((unsigned)((a.N + 16 * WN * WAVES - 1) / (16 * WN * WAVES)),
            (unsigned)((a.M + 16 * WM - 1) / (16 * WM)), (unsigned)(batch * a.parts));
  hipLaunchKernelGGL((k_gemm_mfma<WM, WN, WAVES, KSPLIT, GD, TD, PF, GSPLIT>), grid,
                     dim3(64 * WAVES * KSPLIT * GSPLIT), 0, s, a);
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

// Several parts per workgroup write fp32 nodes only (no bf16 copy, no row
// maxima, no SwiGLU), through a 32-bit buffer range over a tile's rows.
static bool multi_part_ok(const GemmArgs &a, int MT) {
  return a.C != nullptr && a.Cb == nullptr && a.pmax == nullptr && a.glu == 0 &&
         (int64_t)MT * a.ldc * 4 < ((int64_t)1 << 31);
}

template <int WM, int WN, int WAVES_M, int WAVES_N, int S, int NX, bool PIPE, int GS, int U, int GD,
          int TD, int MINB = 1, int PPW = 1>
static int launch_ring_cfg(const GemmArgs &a, hipStream_t s) {
  constexpr int MT = 16 * WM * WAVES_M, NT = 16 * WN * WAVES_N;
  if (a.parts % PPW != 0 || (PPW > 1 && !multi_part_ok(a, MT))) return TBIK_ERR_ARG;
  // the fused row maxima exist for 64-column waves and for 32-column waves
  // four to a tile row only
  if (a.pmax != nullptr && !(WN == 4 || (WN == 2 && WAVES_N == 4))) return TBIK_ERR_ARG;
  TileMap tm;
  tm.tiles_m = (a.M + MT - 1) / MT;
  tm.tiles_n = (a.N + NT - 1) / NT;
  tm.parts = a.parts;
  tm.group_m = 8;
  const int64_t nb = (int64_t)tm.tiles_m * tm.tiles_n * (tm.parts / PPW);
  if (nb > 0x7fffffff) return TBIK_ERR_SHAPE;
  hipLaunchKernelGGL((k_gemm_ring<WM, WN, WAVES_M, WAVES_N, S, NX, PIPE, GS, U, GD, TD, MINB, PPW>),
                     dim3((unsigned)nb), dim3(64 * WAVES_M * WAVES_N), 0, s, a, tm);
  return check_launch();
}

// Tile geometries: "narrow" 128 x 64 (4 waves of 32 x 64 along M, three
// leaf accumulators; the fallback for few tiles and deep group stacks) and
// "wide" 128 x 128 (8 waves of 64 x 32, below) -- the wide tile moves a third
// less data per MFMA.
template <int GS, int U, int GD, int TD>
static int launch_narrow(const GemmArgs &a, hipStream_t s) {
  // fragment pipelining only with the compile-time schedules, whose live
  // state leaves room for the second fragment set
  return launch_ring_cfg<TBIK_RING_WM, TBIK_RING_WN, TBIK_RING_WAVES_M, TBIK_RING_WAVES_N,
                         TBIK_RING_S, TBIK_RING_NX, (TBIK_RING_PIPE != 0 && GS > 0), GS, U, GD, TD>(
      a, s);
}

// One group per part (gpp == 1), or 11-leaf groups, and 2, 4 or 8 parts,
// where the tiles alone give every CU one or two workgroups: a workgroup
// streams all parts of its tile through one ring, writing each part's node
// as soon as it is complete, instead of one short workgroup per part
// (M = 4096, K = N = 2048 at tp = 4, 8 leaves per part: 116 -> 82 us).  With
// more tiles the per-part workgroups were faster (M = N = K = 4096 at
// tp = 4 / 8 and the dp = 8 weight gradient ran 9-15% slower this way).
static bool wide_all_parts(const GemmArgs &a) {
  const int64_t tiles = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
  return TBIK_RING_ALL_PARTS && (a.gpp == 1 || a.G == 11) && multi_part_ok(a, 128) &&
         (a.parts == 2 || a.parts == 4 || a.parts == 8) && tiles >= TBIK_RING_PPW_MIN_WG &&
         tiles <= 2 * TBIK_RING_PPW_MIN_WG;
}

// Reachable (group size, parts): the parts times the groups per part make
// the tree's 8 top groups.  GS = 4 comes with 8 parts (one group each), the
// merged perfect trees GS = 8, 16, 32 with the tp that leaves two or more of
// the original groups in a part, and GS = 11 with any of 2, 4, 8 parts.
template <int GS, int U>
static int launch_wide_all_parts(const GemmArgs &a, hipStream_t s) {
  if constexpr (GS == 11) {
    // 11-leaf groups (K = 5632): 8 / parts groups per part, their own stack
    if (a.parts == 2) return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, 11, 1, 0, 2, 1, 2>(a, s);
    if (a.parts == 4) return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, 11, 1, 0, 1, 1, 4>(a, s);
    if (a.parts == 8) return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, 11, 1, 0, 1, 1, 8>(a, s);
  } else {
    if constexpr (GS != 4) {
      if (a.parts == 2) return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, GS, U, 0, 1, 1, 2>(a, s);
      if (a.parts == 4) return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, GS, U, 0, 1, 1, 4>(a, s);
    }
    if constexpr (GS <= 8)
      if (a.parts == 8) return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, GS, U, 0, 1, 1, 8>(a, s);
  }
  return TBIK_ERR_ARG;
}

// "Wide" tiles: 128 x 128 with 8 waves of 64 x 32, two waves per SIMD (so
// <= 256 registers per wave: two leaf accumulators plus the tree state of
// 32 outputs per lane) and a 4-stage ring of 128 KB.  Against 4 waves of
// 64 x 64 with the same tile (one wave per SIMD, ~460 registers) the copy of
// the operands into LDS runs at nearly twice the rate: the outstanding
// L1 -> L2 requests per CU grow with the resident waves, and the average L2
// latency decides the rate at a given count.
template <int GS, int U = 1>
static int launch_wide(const GemmArgs &a, hipStream_t s) {
  if constexpr (GS == 16 || GS == 32) {
    if (wide_all_parts(a)) return launch_wide_all_parts<GS, U>(a, s);
    if (a.gpp == 1) return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, GS, U, 0, 1, 1>(a, s);
    return TBIK_ERR_ARG;
  } else if constexpr (GS == 28) {
    // at most 4 groups per part (8 would spill the group stack).  One group
    // per part (the tp = 8 shards of a 224-leaf K): two parts per workgroup
    // while that still gives every CU a workgroup.
    if (a.gpp == 1 && a.parts % 2 == 0 && multi_part_ok(a, 128) &&
        (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128) * (a.parts / 2) >= TBIK_RING_PPW_MIN_WG)
      return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, GS, 0, 0, 1, 1, 2>(a, s);
    switch (a.gpp) {
      case 1:
      case 2: return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, GS, 0, 0, 1, 1>(a, s);
      case 4: return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, GS, 0, 0, 2, 1>(a, s);
    }
    return TBIK_ERR_ARG;
  } else {
    if constexpr (GS == 4 || GS == 8 || GS == 11)
      if (wide_all_parts(a)) return launch_wide_all_parts<GS, 1>(a, s);
    switch (a.gpp) {
      case 1:
      case 2: return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, GS, 1, 0, 1, 1>(a, s);
      case 4: return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, GS, 1, 0, 2, 1>(a, s);
      case 8: return launch_ring_cfg<4, 2, 2, 4, 4, 2, false, GS, 1, 0, 3, 1>(a, s);
    }
    return TBIK_ERR_ARG;
  }
}

// "Thin" tiles for M <= 32: 32 x 64 (4 waves of 32 x 16) or, for M <= 16,
// 16 x 64 (2 waves of 16 x 32), on the LDS ring.  With one or two 28-leaf
// groups per part (K split at tree nodes into 4 or 8 parts) a workgroup
// reads only its part's K slice of A, where a small-M kernel over the whole
// K reads all of A once per 16-column block -- at M = 32 twice the bytes of
// W.
#ifndef TBIK_THIN_WN
#define TBIK_THIN_WN 1
#endif
static int launch_thin28(const GemmArgs &a, hipStream_t s) {
  if (a.gpp > 2) return TBIK_ERR_ARG;
  if (a.M <= 16)
    return launch_ring_cfg<1, 2, 1, 2, 4, 2, false, 28, 0, 0, 1, TBIK_THIN_MINB>(a, s);
  return launch_ring_cfg<2, TBIK_THIN_WN, 1, 4, 4, 2, false, 28, 0, 0, 1, TBIK_THIN_MINB>(a, s);
}

template <int GS, int U, int GD>
static int launch_narrow_td(const GemmArgs &a, hipStream_t s) {
  switch (a.gpp) {
    case 1:
    case 2: return launch_narrow<GS, U, GD, 1>(a, s);
    case 4: return launch_narrow<GS, U, GD, 2>(a, s);
    case 8: return launch_narrow<GS, U, GD, 3>(a, s);
  }
  return TBIK_ERR_ARG;
}

static bool ring_supported_g(int G) {
  if (G == 28 || G == 8 || G == 4) return true;
  const int U = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : 1;
  return bit_length(G / U - 1) <= (U == 1 ? 5 : 3);
}

static int launch_ring(const GemmArgs &a, hipStream_t s) {
  const int G = a.G;
  const int64_t wide_tiles = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128) * a.parts;
  if (wide_tiles >= 256) {
    // 128 x 128 tiles, 8 waves: wherever the tree state of a 64 x 32 wave
    // tile fits 256 registers and there are enough tiles for every CU
    if ((G & (G - 1)) == 0 && a.gpp > 1 && G * a.gpp >= 8 && G * a.gpp <= 32) {
      // G a power of two: the part's tree (PAIR of each group = a perfect
      // tree, then the perfect top over gpp groups) is one perfect tree over
      // G * gpp leaves, evaluated as a single compile-time group
      GemmArgs b = a;
      b.G = G * a.gpp;
      b.gpp = 1;
      return b.G == 32 ? launch_wide<32, 0>(b, s)
                       : b.G == 16 ? launch_wide<16, 0>(b, s) : launch_wide<8>(b, s);
    }
    if (G == 4) return launch_wide<4>(a, s);
    if (G == 8) return launch_wide<8>(a, s);
    if (G == 11) return launch_wide<11>(a, s);
    if (G == 28 && a.gpp <= 4) return launch_wide<28>(a, s);
  }
  if (G == 28) return launch_narrow_td<28, 1, 0>(a, s);
  if (G == 11) return launch_narrow_td<11, 1, 0>(a, s);
  if (G == 8) return launch_narrow_td<8, 1, 0>(a, s);
  if (G == 4) return launch_narrow_td<4, 1, 0>(a, s);
  if (G % 8 == 0 && bit_length(G / 8 - 1) <= 3) return launch_narrow_td<0, 8, 3>(a, s);
  if (G % 4 == 0 && bit_length(G / 4 - 1) <= 3) return launch_narrow_td<0, 4, 3>(a, s);
  const int need = bit_length(G - 1);
  if (need <= 3) return launch_narrow_td<0, 1, 3>(a, s);
  if (need <= 5) return launch_narrow_td<0, 1, 5>(a, s);
  return TBIK_ERR_ARG;
}

// Small M: one wave per group of the part, combined in LDS.
template <int WM, int GD>
static int launch_small(const GemmArgs &a, int batch, hipStream_t s) {
  // the split pays for 16-row tiles (M <= 16: +20% at K = 14336); with
  // 32-row tiles the second wave's register tile and LDS exchange cost more
  if (TBIK_SMALL_GSPLIT == 2 && WM == 1 && a.G >= 2) {
    switch (a.gpp) {
      case 1: return launch_cfg<WM, 1, 1, 1, GD, 0, TBIK_SMALL_PF, 2>(a, batch, s);
      case 2: return launch_cfg<WM, 1, 1, 2, GD, 0, TBIK_SMALL_PF, 2>(a, batch, s);
      case 4: return launch_cfg<WM, 1, 1, 4, GD, 0, TBIK_SMALL_PF, 2>(a, batch, s);
      case 8: return launch_cfg<WM, 1, 1, 8, GD, 0, TBIK_SMALL_PF, 2>(a, batch, s);
    }
    return TBIK_ERR_ARG;
  }
  switch (a.gpp) {
    case 1: return launch_cfg<WM, 1, 1, 1, GD, 0, TBIK_SMALL_PF>(a, batch, s);
    case 2: return launch_cfg<WM, 1, 1, 2, GD, 0, TBIK_SMALL_PF>(a, batch, s);
    case 4: return launch_cfg<WM, 1, 1, 4, GD, 0, TBIK_SMALL_PF>(a, batch, s);
    case 8: return launch_cfg<WM, 1, 1, 8, GD, 0, TBIK_SMALL_PF>(a, batch, s);
  }
  return TBIK_ERR_ARG;
}

// Number of aligned tree nodes (1, 2, 4 or 8 parts) into which tbik_gemm
// splits K when a workspace is given (the split is at node boundaries, so the
// bits do not change).  28-leaf groups (K = 14336): the wide tiles hold at
// most 4 groups per part without spilling, so at least 2 parts, and more
// until the wide tiles fill every CU.  Otherwise the smallest split that
// gives the ring kernel about one 128 x 64 workgroup per CU.  1 = no split
// (small M, batched, scalar leaves, or enough tiles).
int gemm_split_parts(int M, int N, int K, int batch, int leaf_mode) {
  if (leaf_mode != TBIK_LEAF_MFMA || batch != 1 || M <= TBIK_THIN_MIN_M || N <= 0 || K <= 0) return 1;
  const int nb = K / 64;
  const int T = tree_T(nb);
  if (M <= 32) return (TBIK_THIN && T == 8 && nb / T == 28) ? 8 : 1;   // thin tiles, one group per part
  if (!ring_supported_g(nb / T)) return 1;
  if (nb / T == 28 && T == 8) {
    const int64_t wide = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
    int p = TBIK_SPLIT28_MIN;
    while (p < T && wide * p < 256) p <<= 1;
    return p;
  }
  const int64_t narrow = (int64_t)((M + 127) / 128) * ((N + 63) / 64);
  for (int p = 1; p <= T; p <<= 1)
    if (narrow * p >= 256) return p;
  return T;
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
  a.pmax = nullptr; a.ld_pmax = 0;
  a.H = c.H; a.ldh = c.ldh; a.glu = c.glu;
  a.gpp = T / (c.shard_of > 0 ? c.shard_of : c.parts);
  if (a.G > kMaxGroupLeaves) return TBIK_ERR_SHAPE;
  if ((int64_t)c.batch * c.parts > 65535) return TBIK_ERR_SHAPE;
  if (c.leaf_mode == TBIK_LEAF_SCALAR && c.M > 65535) return TBIK_ERR_SHAPE;
  if ((c.M + 15) / 16 > 65535) return TBIK_ERR_SHAPE;
  if (c.pmax) {
    // row maxima: fused into the ring kernel's epilogue where it runs,
    // otherwise a pass over C after the GEMM
    const bool ring = c.leaf_mode == TBIK_LEAF_MFMA && c.M > 32 && c.batch == 1 &&
                      c.parts == 1 && c.shard_of == 0 && ring_supported_g(nb / T) &&
                      (int64_t)128 * c.lda * 2 < ((int64_t)1 << 31) &&
                      (int64_t)128 * c.ldw * 2 < ((int64_t)1 << 31);
    if (ring) {
      a.pmax = c.pmax; a.ld_pmax = c.ld_pmax;
      return launch_ring(a, s);
    }
    GemmCall c2 = c;
    c2.pmax = nullptr;
    const int rc = launch_gemm(c2, s);
    if (rc) return rc;
    return launch_block_rowmax(c.C, c.ldc, c.M, c.N, c.pmax, c.ld_pmax, s);
  }
  if (c.glu) {
    // SwiGLU epilogue: the ring kernel on the whole tree (one part, one
    // batch), W addressed through one 32-bit buffer range
    if (c.leaf_mode != TBIK_LEAF_MFMA || c.M <= 32 || c.batch != 1 || c.parts != 1 ||
        c.shard_of != 0 || (c.N % 32) != 0 || !ring_supported_g(a.G) ||
        (int64_t)128 * c.lda * 2 >= ((int64_t)1 << 31) ||
        (int64_t)c.N * c.ldw * 2 >= ((int64_t)1 << 31))
      return TBIK_ERR_SHAPE;
    return launch_ring(a, s);
  }
  if (c.leaf_mode == TBIK_LEAF_SCALAR) {
    dim3 grid((unsigned)((c.N + 63) / 64), (unsigned)c.M, (unsigned)(c.batch * c.parts));
    hipLaunchKernelGGL(k_gemm_scalar, grid, dim3(64), 0, s, a);
    return check_launch();
  }
  const int need = bit_length(a.G - 1);
  if (TBIK_THIN && c.M > TBIK_THIN_MIN_M && c.M <= 32 && c.batch == 1 && a.G == 28 && a.gpp <= 2 &&
      (int64_t)32 * c.lda * 2 < ((int64_t)1 << 31) && (int64_t)128 * c.ldw * 2 < ((int64_t)1 << 31))
    return launch_thin28(a, s);
  if (c.M > 32 && c.batch == 1 && ring_supported_g(a.G) &&
      (int64_t)128 * c.lda * 2 < ((int64_t)1 << 31) && (int64_t)128 * c.ldw * 2 < ((int64_t)1 << 31))
    return launch_ring(a, s);
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
  const bool vec = (N % 4) == 0 && (ldc % 4) == 0 && ((uintptr_t)ws & 15) == 0 &&
                   (!C || ((uintptr_t)C & 15) == 0) && (!Cb || ((uintptr_t)Cb & 7) == 0);
  if (vec) {
    int64_t blocks = (mn / 4 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    dim3 grid((unsigned)blocks), block(256);
    switch (tp) {
      case 1: hipLaunchKernelGGL(k_tree_combine4<1>, grid, block, 0, s, ws, mn, N, C, Cb, ldc); break;
      case 2: hipLaunchKernelGGL(k_tree_combine4<2>, grid, block, 0, s, ws, mn, N, C, Cb, ldc); break;
      case 4: hipLaunchKernelGGL(k_tree_combine4<4>, grid, block, 0, s, ws, mn, N, C, Cb, ldc); break;
      case 8: hipLaunchKernelGGL(k_tree_combine4<8>, grid, block, 0, s, ws, mn, N, C, Cb, ldc); break;
      default: return TBIK_ERR_TP;
    }
    return check_launch();
  }
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
