// tbik_device.h -- device-side numerics of libtbik (gfx950).
//
// bf16 rounding, the library-defined EXP/LOG, and the streaming form of the
// reduction tree.  Written for this library only; the CPU oracle used by the
// tests is an independent implementation of the same definitions.
//
// Every floating-point operation here must be one IEEE binary32 operation:
// the library is compiled with -ffp-contract=off, without fast-math, with
// IEEE denormals and correctly rounded fp32 divide/sqrt.  Hardware
// transcendental instructions (v_exp_f32, v_log_f32, v_rsq_f32) are never
// used.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

namespace tbik {

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest, ties to even, subnormals kept: the gfx950
// conversion instruction (v_cvt_pk_bf16_f32) under the default rounding mode
// with fp32 denormals enabled.  A NaN becomes a quiet NaN of the same sign
// (its payload is not specified).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two conversions in one instruction: a in the low half, b in the high half.
// v rounded to the nearest bf16 and widened back: one bf16 operation of
// eager bf16 arithmetic (the misaligned rounding location of a node)
__device__ __forceinline__ float bf_round(float v) { return bf2f(f2bf(v)); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// --- EXP ---------------------------------------------------------------------
// x = k ln2 + r, k = rint(x log2 e); r via two fma with ln2 split into
// hi (ln2 rounded to a multiple of 2^-16, so k*hi is exact for |k| < 2^8)
// and lo; e^r by the degree-7 Taylor polynomial (coefficients 1/n! rounded
// to fp32) in Horner form with fma; 2^k applied with one rounding.  The
// definition applies 2^k as two power-of-two multiplies (2^floor(k/2), then
// 2^(k - floor(k/2))), whose first product is exact; v_ldexp_f32 rounds
// p * 2^k once as well, and the two agree bit for bit on every fp32 input
// (checked exhaustively on the GPU), in one instruction instead of six.
//
// EXP's special cases (x > 89 -> +inf, x < -104 -> +0) need no branch or
// select: with x clamped to [-104.5, 89.5] the main path itself overflows
// to +inf above 89 and rounds to +0 below -104, and inside [-104, 89] the
// clamp is the identity.  This equality holds for every non-NaN fp32 x (an
// exhaustive check of all 2^32 inputs).
__device__ __forceinline__ float exp_clamp(float x) {
  return __builtin_fminf(__builtin_fmaxf(x, -104.5f), 89.5f);
}

// Main path; x must lie in [-104.5, 89.5].
__device__ __forceinline__ float exp_core(float x) {
  const float kf = __builtin_rintf(x * 0x1.715476p+0f);
  const int k = (int)kf;
  float r = __builtin_fmaf(-kf, 0x1.62e4p-1f, x);
  r = __builtin_fmaf(-kf, 0x1.7f7d1cp-20f, r);
  float p = 0x1.a01a02p-13f;                   // 1/7!
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);   // 1/6!
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);    // 1/5!
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);    // 1/4!
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);    // 1/3!
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, k);
}

// EXP of any fp32 x; a NaN is returned quieted (x + x).
__device__ __forceinline__ float exp_f32(float x) {
  const float res = exp_core(exp_clamp(x));
  return (x != x) ? x + x : res;
}

// --- SiLU ---------------------------------------------------------------------
// silu(g) = g / (1 + EXP(-g)), the division correctly rounded.
// Fast path: the quotient from a refined reciprocal plus one exact-remainder
// correction (Markstein's scheme).  The gate is bf16, so silu has only
// 2^16 possible arguments: for every finite bf16 g with g >= -87 and
// |g| >= 2^-20 the fast path returns the IEEE quotient, whatever reciprocal
// within 3 ulp the hardware's v_rcp_f32 gives (checked exhaustively on the
// CPU for each such reciprocal; the GPU path is checked against the oracle on
// all 2^16 gates).  g >= -87 keeps 1 + EXP(-g) below 2^126, so the reciprocal
// is a normal number.  Every other g (NaN, +-inf, g < -87, tiny |g|) takes
// the IEEE division in a branch that random activations essentially never
// enter.
__device__ __forceinline__ float silu_den(float g) { return 1.0f + exp_core(exp_clamp(-g)); }

__device__ __forceinline__ bool silu_fast_ok(float g) {
  return g >= -87.0f && __builtin_fabsf(g) >= 0x1p-20f && g <= 0x1.fffffep+127f;
}

__device__ __forceinline__ float silu_fast(float g, float d) {
  const float y0 = __builtin_amdgcn_rcpf(d);
  const float e0 = __builtin_fmaf(-d, y0, 1.0f);
  const float y1 = __builtin_fmaf(e0, y0, y0);
  const float q0 = g * y1;
  const float rm = __builtin_fmaf(-d, q0, g);
  return __builtin_fmaf(rm, y1, q0);
}

// n gates at once; the IEEE fallback is one branch for all n.
template <int n>
__device__ __forceinline__ void silu_n(float (&g)[n]) {
  float d[n];
  bool slow = false;
#pragma unroll
  for (int e = 0; e < n; ++e) {
    d[e] = silu_den(g[e]);
    slow = slow || !silu_fast_ok(g[e]);
  }
  if (slow) {
#pragma unroll
    for (int e = 0; e < n; ++e) g[e] = silu_fast_ok(g[e]) ? silu_fast(g[e], d[e]) : g[e] / d[e];
  } else {
#pragma unroll
    for (int e = 0; e < n; ++e) g[e] = silu_fast(g[e], d[e]);
  }
}

__device__ __forceinline__ float silu(float g) {
  float v[1] = {g};
  silu_n<1>(v);
  return v[0];
}

// --- LOG ---------------------------------------------------------------------
// x = 2^k m, m in [sqrt(1/2), sqrt(2)); f = m - 1 (exact); s = f/(2+f);
// log(1+f) = 2 atanh(s) = f - hfsq + s (hfsq + R(s^2)), hfsq = f^2/2,
// R(z) = 2z/3 + 2z^2/5 + 2z^3/7 + 2z^4/9; then + k ln2 with the split ln2.
__device__ __forceinline__ float log_f32(float x) {
  if (x != x) return x + x;
  if (x < 0.0f) return __builtin_nanf("");
  if (x == 0.0f) return -__builtin_inff();
  if (x == __builtin_inff()) return x;
  uint32_t ix = __float_as_uint(x);
  int k = 0;
  if (ix < 0x00800000u) {                 // subnormal: scale by 2^25
    x = x * 0x1p25f;
    ix = __float_as_uint(x);
    k = -25;
  }
  k += (int)(ix >> 23) - 127;
  const uint32_t mant = ix & 0x007fffffu;
  float m;
  if (mant > 0x3504f3u) {                 // mantissa above that of fp32(sqrt 2)
    m = __uint_as_float(mant | 0x3f000000u);
    k += 1;
  } else {
    m = __uint_as_float(mant | 0x3f800000u);
  }
  const float f = m - 1.0f;
  const float s = f / (2.0f + f);
  const float z = s * s;
  float R = __builtin_fmaf(z, 0x1.c71c72p-3f, 0x1.24924ap-2f);   // 2/9, 2/7
  R = __builtin_fmaf(z, R, 0x1.99999ap-2f);                       // 2/5
  R = __builtin_fmaf(z, R, 0x1.555556p-1f);                       // 2/3
  R = z * R;
  const float hfsq = (0.5f * f) * f;
  const float kf = (float)k;
  return kf * 0x1.62e4p-1f - ((hfsq - (s * (hfsq + R) + kf * 0x1.7f7d1cp-20f)) - f);
}

// --- the tree ----------------------------------------------------------------
// T of the tree over n leaves: the largest power of two <= 8 dividing n.
__host__ __device__ __forceinline__ int tree_T(int64_t n) {
  int T = 8;
  while (T > 1 && (n % T) != 0) T >>= 1;
  return T;
}

// Streaming evaluation of one PAIR reduction over n leaves that arrive in
// order (index cnt = 0, 1, ...), R values per lane at once (a register tile).
// s[j] holds the finished subtree of 2^j leaves at level j.  The merge of a
// new leaf is a binary-counter carry (levels below the trailing-ones count
// of cnt); the last leaf folds the remaining subtrees in from the lowest to
// the highest level.  That is PAIR's structure: a left-to-right sequence of
// power-of-two blocks, block j+1 added to the fold of the smaller blocks.
// D must be at least the bit length of n-1.  cnt and n are wave-uniform, so
// every branch below is a scalar branch and every index is static.
// Returns true on the last leaf; the PAIR value is then in `node`.
template <int R, int D>
__device__ __forceinline__ bool pair_push(float (&s)[D > 0 ? D : 1][R], float (&node)[R], int cnt,
                                          int n) {
  const int t = __builtin_ctz(~(unsigned)cnt);
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if (j < t) {
#pragma unroll
      for (int r = 0; r < R; ++r) node[r] = s[j][r] + node[r];
    }
  }
  if (cnt + 1 == n) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (j > t && ((cnt >> j) & 1)) {
#pragma unroll
        for (int r = 0; r < R; ++r) node[r] = s[j][r] + node[r];
      }
    }
    return true;
  }
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if (j == t) {
#pragma unroll
      for (int r = 0; r < R; ++r) s[j][r] = node[r];
    }
  }
  return false;
}

// Bit length of v (0 for v == 0).
__host__ __device__ __forceinline__ int bit_length(int64_t v) {
  int b = 0;
  while (v > 0) { ++b; v >>= 1; }
  return b;
}

}  // namespace tbik
