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
// query rows and all Lk keys.  MFMA accumulator lane l, register i holds
// row 4(l/16)+i, column l%16 of a 16x16 block.
#include "tbik_device.h"
#include "tbik_internal.h"
#include "../../include/tbik.h"

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

}  // namespace

template <int LK>
__global__ void __launch_bounds__(256)
k_attn_causal(const uint16_t *Q, int64_t ldq, const uint16_t *K, int64_t ldk, const uint16_t *Vt,
              int64_t ldvt, uint16_t *O, int64_t ldo, int heads, float scale) {
  constexpr int HD = 128;
  constexpr int NB = LK / 16;          // 16-key blocks
  constexpr int NL = LK / 64;          // 64-key leaves of P V
  __shared__ u32x4 pl[4][16][LK / 8];  // P rows of each wave, bf16
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y % heads, b = blockIdx.y / heads;
  const int r0 = blockIdx.x * 64 + wave * 16;        // first query row of this wave
  const int64_t tok0 = (int64_t)b * LK;
  const int lr = lane & 15, lk = (lane >> 4) * 8;

  // ---- S = Q K^T for the wave's 16 rows and all keys
  u32x4 qa[2][2];
  {
    const uint16_t *qp = Q + (tok0 + r0 + lr) * ldq + (int64_t)h * HD + lk;
#pragma unroll
    for (int lf = 0; lf < 2; ++lf)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qa[lf][hf] = *reinterpret_cast<const u32x4 *>(qp + 64 * lf + 32 * hf);
  }
  float s[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint16_t *kp = K + (tok0 + nb * 16 + lr) * ldk + (int64_t)h * HD + lk;
    u32x4 kb[2][2];
#pragma unroll
    for (int lf = 0; lf < 2; ++lf)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        kb[lf][hf] = *reinterpret_cast<const u32x4 *>(kp + 64 * lf + 32 * hf);
    const f32x4 l0 = mfma2(qa[0][0], kb[0][0], qa[0][1], kb[0][1]);
    const f32x4 l1 = mfma2(qa[1][0], kb[1][0], qa[1][1], kb[1][1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[nb][i] = l0[i] + l1[i];
  }

  // ---- causal softmax per row: row 4(l/16)+i, key 16 nb + l%16
  const int rowb = r0 + 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rowb + i;
    float m = -__builtin_inff();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s[nb][i] = s[nb][i] * scale;
      if (nb * 16 + lr <= row) m = __builtin_fmaxf(m, s[nb][i]);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb][i] = (nb * 16 + lr <= row) ? exp_f32(s[nb][i] - m) : 0.0f;
    // perfect tree over the keys: the 16 columns of a block across lanes
    // (xor 1, 2, 4, 8 pairs neighbouring columns), then the blocks in-lane
    float blk[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float v = s[nb][i];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) v = v + __shfl_xor(v, off);
      blk[nb] = v;
    }
#pragma unroll
    for (int w = NB; w > 1; w >>= 1)
#pragma unroll
      for (int q = 0; q < w / 2; ++q) blk[q] = blk[2 * q] + blk[2 * q + 1];
    const float ssum = blk[0];
    uint16_t *prow = reinterpret_cast<uint16_t *>(&pl[wave][4 * (lane >> 4) + i][0]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float p = (nb * 16 + lr <= row) ? s[nb][i] / ssum : 0.0f;
      prow[nb * 16 + lr] = f2bf(p);
    }
  }
  __syncthreads();

  // ---- O = P V: leaves of 64 keys, perfect tree over the NL leaves
  float node[8][4];
  float st[4][8][4];                   // perfect-tree stack (NL <= 8)
#pragma unroll
  for (int kl = 0; kl < NL; ++kl) {
    u32x4 pa[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) pa[hf] = pl[wave][lr][(64 * kl + 32 * hf + lk) / 8];
    float leaf[8][4];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const uint16_t *vp = Vt + ((int64_t)h * HD + nb * 16 + lr) * ldvt + tok0 + 64 * kl + lk;
      const u32x4 v0 = *reinterpret_cast<const u32x4 *>(vp);
      const u32x4 v1 = *reinterpret_cast<const u32x4 *>(vp + 32);
      const f32x4 acc = mfma2(pa[0], v0, pa[1], v1);
#pragma unroll
      for (int i = 0; i < 4; ++i) leaf[nb][i] = acc[i];
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
  const dim3 grid((unsigned)(L / 64), (unsigned)(heads * batch)), block(256);
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
