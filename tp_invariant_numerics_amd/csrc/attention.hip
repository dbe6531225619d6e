// attention.hip -- fused invariant causal attention (decoder composition).
//
// For one (sequence, head) it returns bit for bit what the unfused
// composition returns:
//   S = tbik_gemm(Q, K)                 K = head_dim = 128: two 64-wide leaves,
//                                       the tree over T = 2 groups: leaf0 + leaf1
//   P = causal softmax of S * scale     max over visible keys, EXP, the tree over
//                                       the Lk keys, one division, P -> bf16
//   O = bf16(tbik_gemm(P, V^T))         Lk/64 leaves over the keys
// (TBIK summary page, "technical framework": the invariant kernels inside the
// model; the causal softmax is the decoder's own glue).  For Lk a power of two
// (64 .. 512) every level of every tree above is a perfect binary tree, so an
// evaluation that pairs the same siblings in any arrangement of lanes and
// registers gives the same bits; the MFMA leaves use the same instruction and
// operand mapping as the GEMM kernels.  No score matrix goes to HBM.
//
// Workgroup = 4 waves = 64 query rows of one (sequence, head); wave w owns 16
// query rows.  Each 64-key chunk of K and of V^T is read from HBM once per
// workgroup into LDS and shared by the four waves; chunks past the
// workgroup's diagonal hold only masked keys and are skipped (their zeros
// still enter the trees at their places, so the bits do not change).  MFMA
// accumulator lane l, register i holds row 4(l/16)+i, column l%16 of a
// 16x16 block.
#include "tbik_device.h"
#include "tbik_internal.h"
#include "../../include/tbik.h"

#ifndef TBIK_ATTN_MINB
#define TBIK_ATTN_MINB 2
#endif

namespace tbik {

namespace {

__device__ __forceinline__ f32x4 mfma2(const u32x4 &a0, const u32x4 &b0, const u32x4 &a1,
                                       const u32x4 &b1) {
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0),
                                                __builtin_bit_cast(bf16x8, b0), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1),
                                                __builtin_bit_cast(bf16x8, b1), acc, 0, 0, 0);
  return acc;
}

// src of another lane of the same 16-lane row, by a DPP pattern:
// 0xB1 / 0x4E quad permutations [1,0,3,2] / [2,3,0,1] (lane ^ 1, lane ^ 2);
// 0x121..0x12F rotate right by 1..15 (lane i reads lane (i - k) mod 16).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Perfect tree over the 16 lanes of a row (lane = column): levels 1-2 pair
// lanes ^1 and ^2 (every lane gets its quad's sum), levels 3-4 add the
// quad 4 and then 8 lanes below (mod 16), which pairs quads (0,1), (2,3)
// in lanes 4-7 and 12-15 and then the two halves there.  Only lanes with
// bit 2 set hold the block sum afterwards.
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp<0xB1>(v);
  v = v + dpp<0x4E>(v);
  v = v + dpp<0x124>(v);
  v = v + dpp<0x128>(v);
  return v;
}

}  // namespace

template <int LK>
__global__ void __launch_bounds__(256, TBIK_ATTN_MINB)
k_attn_causal(const uint16_t *Q, int64_t ldq, const uint16_t *K, int64_t ldk, const uint16_t *Vt,
              int64_t ldvt, uint16_t *O, int64_t ldo, int heads, float scale) {
  constexpr int HD = 128;
  constexpr int NB = LK / 16;          // 16-key blocks
  constexpr int NL = LK / 64;          // 64-key chunks = leaves of P V
  constexpr int PC = LK / 8;           // 16-byte chunks per P row
  constexpr int PSW = (PC < 16 ? PC : 16) - 1;   // P swizzle mask: stays inside the row
  // LDS: one 16 KB tile that holds the current K chunk [64 keys][128 dims]
  // during S and the current V^T chunk [128 dims][64 keys] during P V, and
  // the P rows of each wave [16][LK].  16-byte chunks are XOR-swizzled by
  // row so that the 16 rows one fragment read touches fall in distinct
  // banks; 80 KB in all for LK = 512, two workgroups per CU.
  __shared__ u32x4 tile[1024];
  __shared__ u32x4 pl[4][16 * PC];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  // grid (sequence x head, row block): every (sequence, head)'s longest row
  // block is dispatched before any shorter one -- longest first packs the
  // causal triangle's unequal workgroups (8:1 at 512 keys) onto the CUs
  const int xb = gridDim.y - 1 - blockIdx.y;
  const int h = blockIdx.x % heads, b = blockIdx.x / heads;
  const int r0 = xb * 64 + wave * 16;          // first query row of this wave
  const int nkc = xb + 1;                      // chunks holding a visible key
  const int64_t tok0 = (int64_t)b * LK;
  const int lr = lane & 15, lg = lane >> 4, lk = lg * 8;
  u32x4 *pw = pl[wave];

  // ---- S = Q K^T for the wave's 16 rows over the visible chunks; the K
  //      chunk is staged in LDS once for the four waves.  Chunks past the
  //      diagonal hold no visible key and are not computed.
  u32x4 qa[2][2];
  {
    const uint16_t *qp = Q + (tok0 + r0 + lr) * ldq + (int64_t)h * HD + lk;
#pragma unroll
    for (int lf = 0; lf < 2; ++lf)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qa[lf][hf] = *reinterpret_cast<const u32x4 *>(qp + 64 * lf + 32 * hf);
  }
  // chunk loads: K chunk kc row (tid >> 4) + 16 i, dims 8 (tid & 15) ..;
  // V^T chunk kl dim (tid >> 3) + 32 i, keys 64 kl + 8 (tid & 7) ..
  auto load_k = [&](u32x4 (&r)[4], int kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = *reinterpret_cast<const u32x4 *>(K + (tok0 + kc * 64 + (tid >> 4) + 16 * i) * ldk +
                                              (int64_t)h * HD + (tid & 15) * 8);
  };
  auto load_v = [&](u32x4 (&r)[4], int kl) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = *reinterpret_cast<const u32x4 *>(Vt + ((int64_t)h * HD + (tid >> 3) + 32 * i) * ldvt +
                                              tok0 + 64 * kl + (tid & 7) * 8);
  };
  u32x4 ld4[4];                                // the next chunk, in flight
  load_k(ld4, 0);
  float s[NB][4];
#pragma unroll
  for (int kc = 0; kc < NL; ++kc) {
    if (kc < nkc) {                            // uniform over the workgroup
      __syncthreads();                         // the previous chunk is consumed
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 4) + 16 * i;   // key; 16 chunks of 8 dims per row
        tile[row * 16 + ((tid & 15) ^ (row & 15))] = ld4[i];
      }
      __syncthreads();
      if (kc + 1 < nkc) load_k(ld4, kc + 1);
      else load_v(ld4, 0);                     // first V^T chunk, during the softmax
#pragma unroll
      for (int n4 = 0; n4 < 4; ++n4) {
        const u32x4 *kp = &tile[(n4 * 16 + lr) * 16];
        u32x4 kb[2][2];
#pragma unroll
        for (int lf = 0; lf < 2; ++lf)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            kb[lf][hf] = kp[(8 * lf + 4 * hf + lg) ^ lr];
        const f32x4 l0 = mfma2(qa[0][0], kb[0][0], qa[0][1], kb[0][1]);
        const f32x4 l1 = mfma2(qa[1][0], kb[1][0], qa[1][1], kb[1][1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kc * 4 + n4][i] = l0[i] + l1[i];
      }
    } else {
#pragma unroll
      for (int n4 = 0; n4 < 4; ++n4)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kc * 4 + n4][i] = 0.0f;
    }
  }

  // ---- causal softmax per row: row 4(l/16)+i, key 16 nb + l%16.  A key
  //      block past the diagonal contributes EXP-free zeros, exactly what
  //      the masked entries of the full row contribute.
  const int rowb = r0 + 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rowb + i;
    float m = -__builtin_inff();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (nb < 4 * nkc) {
        s[nb][i] = s[nb][i] * scale;
        if (nb * 16 + lr <= row) m = __builtin_fmaxf(m, s[nb][i]);
      }
    }
    // exact maximum over the row's 16 lanes (rotations by 1, 2, 4, 8)
    m = __builtin_fmaxf(m, dpp<0x121>(m));
    m = __builtin_fmaxf(m, dpp<0x122>(m));
    m = __builtin_fmaxf(m, dpp<0x124>(m));
    m = __builtin_fmaxf(m, dpp<0x128>(m));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      s[nb][i] = (nb < 4 * nkc && nb * 16 + lr <= row) ? exp_f32(s[nb][i] - m) : 0.0f;
    // perfect tree over the keys: the 16 columns of a block across lanes
    // (row16_sum), then the blocks in-lane; lanes 4-7 and 12-15 of the row
    // finish it and pass the sum to the lanes 4 below them (mod 16)
    float blk[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) blk[nb] = nb < 4 * nkc ? row16_sum(s[nb][i]) : 0.0f;
#pragma unroll
    for (int w = NB; w > 1; w >>= 1)
#pragma unroll
      for (int q = 0; q < w / 2; ++q) blk[q] = blk[2 * q] + blk[2 * q + 1];
    // one DPP move with bank mask 0b0101: lanes 0-3 and 8-11 take the value
    // of the lanes 4 below them (mod 16), lanes 4-7 and 12-15 keep theirs
    // (no branch: a DPP read of lanes switched off by a branch gives 0)
    const float ssum = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, blk[0]),
                                           __builtin_bit_cast(int, blk[0]), 0x124, 0xf, 0x5, false));
    const int prw = 4 * (lane >> 4) + i;      // row of the wave's P
    uint16_t *prow = reinterpret_cast<uint16_t *>(pw + prw * PC);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (nb < 4 * nkc) {
        const float p = (nb * 16 + lr <= row) ? s[nb][i] / ssum : 0.0f;
        const int e = nb * 16 + lr;            // key; chunk e / 8 swizzled by the row
        prow[(((e >> 3) ^ (prw & PSW)) << 3) | (e & 7)] = f2bf(p);
      }
    }
  }

  // ---- O = P V: leaves of 64 keys (one V^T chunk in LDS each), perfect
  //      tree over the NL leaves; a leaf past the diagonal is +0, the value
  //      of a leaf whose P entries are all zero.
  float node[8][4];
  float st[4][8][4];                   // perfect-tree stack (NL <= 8)
#pragma unroll
  for (int kl = 0; kl < NL; ++kl) {
    float leaf[8][4];
    if (kl < nkc) {
      __syncthreads();                         // previous chunk consumed; P visible
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = (tid >> 3) + 32 * i;     // dim; 8 chunks of 8 keys per row
        tile[d * 8 + ((tid & 7) ^ ((d >> 1) & 7))] = ld4[i];
      }
      __syncthreads();
      if (kl + 1 < nkc) load_v(ld4, kl + 1);
      u32x4 pa[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) pa[hf] = pw[lr * PC + ((8 * kl + 4 * hf + lg) ^ (lr & PSW))];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int d = nb * 16 + lr;
        const u32x4 v0 = tile[d * 8 + (lg ^ ((d >> 1) & 7))];
        const u32x4 v1 = tile[d * 8 + ((4 + lg) ^ ((d >> 1) & 7))];
        const f32x4 acc = mfma2(pa[0], v0, pa[1], v1);
#pragma unroll
        for (int i = 0; i < 4; ++i) leaf[nb][i] = acc[i];
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) leaf[nb][i] = 0.0f;
    }
    // binary-counter merge: leaf kl joins the subtrees of the set low bits
    int lvl = 0;
    for (int c = kl; c & 1; c >>= 1, ++lvl) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) leaf[nb][i] = st[lvl][nb][i] + leaf[nb][i];
    }
    if (kl == NL - 1) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) node[nb][i] = leaf[nb][i];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q == lvl) {
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) st[q][nb][i] = leaf[nb][i];
        }
    }
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      O[(tok0 + rowb + i) * ldo + (int64_t)h * HD + nb * 16 + lr] = f2bf(node[nb][i]);
}

int launch_attn_causal(const uint16_t *Q, int64_t ldq, const uint16_t *K, int64_t ldk,
                       const uint16_t *Vt, int64_t ldvt, uint16_t *O, int64_t ldo, int L, int heads,
                       int batch, float scale, hipStream_t s) {
  const dim3 grid((unsigned)(heads * batch), (unsigned)(L / 64)), block(256);
  switch (L) {
    case 64: hipLaunchKernelGGL(k_attn_causal<64>, grid, block, 0, s, Q, ldq, K, ldk, Vt, ldvt, O, ldo, heads, scale); break;
    case 128: hipLaunchKernelGGL(k_attn_causal<128>, grid, block, 0, s, Q, ldq, K, ldk, Vt, ldvt, O, ldo, heads, scale); break;
    case 256: hipLaunchKernelGGL(k_attn_causal<256>, grid, block, 0, s, Q, ldq, K, ldk, Vt, ldvt, O, ldo, heads, scale); break;
    case 512: hipLaunchKernelGGL(k_attn_causal<512>, grid, block, 0, s, Q, ldq, K, ldk, Vt, ldvt, O, ldo, heads, scale); break;
    default: return TBIK_ERR_SHAPE;
  }
  return hipGetLastError() == hipSuccess ? TBIK_OK : TBIK_ERR_LAUNCH;
}

}  // namespace tbik
