// rowops.hip -- TP-invariant row reductions and fp32-intermediate nodes.
//
//  * residual-add + RMSNorm, RoPE, SwiGLU: fp32 intermediates, one bf16
//    rounding at the output (rounding-alignment article, "three nodes").
//  * log-softmax + target gather and the causal softmax: the row sum
//    follows the library's tree (TBIK summary page, Abstract: TP-invariant
//    reduction primitives); the vocab groups of the tree are the shards of
//    a vocab-parallel layout.
//
// Row trees are evaluated in three stages that reproduce the same PAIR
// structure: (1) each thread reduces an aligned chunk of CH = 2^c leaves
// (2^c divides the group size, so PAIR's first c levels are perfect trees
// over exactly these chunks); (2) PAIR's remaining levels run level by level
// in LDS (ping-pong buffers, one barrier per level, odd last element carried);
// (3) the perfect tree over the T group sums.  When the group size has too
// few factors of two for such chunks to fit LDS, the *_tail kernels use
// 16-leaf chunks plus one tail item per group (TailRows), the same tree.
// No atomics.
#include "tbik_device.h"
#include "tbik_internal.h"
#include "../../include/tbik.h"

namespace tbik {

static int check_launch() {
  return hipGetLastError() == hipSuccess ? TBIK_OK : TBIK_ERR_LAUNCH;
}

template <int CH>
__device__ __forceinline__ float chunk_tree(float (&v)[CH]) {
#pragma unroll
  for (int w = CH; w > 1; w >>= 1) {
#pragma unroll
    for (int q = 0; q < w / 2; ++q) v[q] = v[2 * q] + v[2 * q + 1];
  }
  return v[0];
}

// PAIR levels over `groups` independent groups of m values each, stored
// compactly (group g at src[g*m .. g*m+m)).  Leaves each group's PAIR value
// at src'[g] (returned pointer).  groups is a power of two dividing NT: each
// group gets NT/groups threads (no division in the index arithmetic).  Must
// be called by all threads of the block.
template <int NT>
__device__ __forceinline__ float *lds_pair(float *src, float *dst, int m, int groups) {
  const int sh = __builtin_ctz((unsigned)(NT / groups));
  const int g = threadIdx.x >> sh, r = threadIdx.x & ((1 << sh) - 1);
  while (m > 1) {
    const int half = m >> 1;
    const int nm = half + (m & 1);
    const float *sg = src + g * m;
    for (int i = r; i < nm; i += 1 << sh)
      dst[g * nm + i] = (i < half) ? sg[2 * i] + sg[2 * i + 1] : sg[m - 1];
    __syncthreads();
    float *t = src; src = dst; dst = t;
    m = nm;
  }
  return src;
}

// Root of the row tree given nch = T*gc chunk values in buf_a (visible to
// all threads).  buf_b is scratch of the same size.
template <int NT>
__device__ __forceinline__ float lds_row_tree(float *buf_a, float *buf_b, int gc, int T) {
  float *g = lds_pair<NT>(buf_a, buf_b, gc, T);
  float *other = (g == buf_a) ? buf_b : buf_a;
  float *root = lds_pair<NT>(g, other, T, 1);
  return root[0];
}

// ---- rows whose groups are not whole chunks -----------------------------------
// A group of G = 16q + r leaves (r < 16): PAIR over it is the right fold of
// perfect trees over the binary decomposition of G, whose blocks of 16 and
// more are perfect trees over aligned 16-leaf chunks.  So it equals PAIR
// over the sequence of q + (r > 0) items -- the q chunk trees, then PAIR over
// the r tail leaves -- appending the tail's value carries through the low
// blocks exactly as the low bits of G do.  This lets a row whose G has few
// factors of two (so that whole-group chunks would be 1 or 2 leaves wide)
// stage about G/16 values per group.
struct TailRows {
  int G, q, r, gs;
  __device__ __forceinline__ TailRows(int n, int T)
      : G(n / T), q((n / T) >> 4), r((n / T) & 15), gs(((n / T) >> 4) + (((n / T) & 15) ? 1 : 0)) {}
  // item `it` (group it / gs): first leaf and leaf count
  __device__ __forceinline__ void item(int it, int &start, int &len) const {
    const int g = it / gs, k = it - g * gs;
    start = g * G + 16 * k;
    len = k < q ? 16 : r;
  }
};

// PAIR over v[0..n), 1 <= n <= 16: neighbours added level by level, an odd
// last element carried up unchanged (for n = 16 the perfect tree).
__device__ __forceinline__ float pair16(float (&v)[16], int n) {
  if (n == 16) return chunk_tree<16>(v);
#pragma unroll
  for (int lev = 0; lev < 4; ++lev) {
    if (n > 1) {
      float last = 0.0f;                         // v[n - 1], read by static indices
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (e == n - 1) last = v[e];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n / 2) v[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((n & 1) && i == n / 2) v[i] = last;
      n = (n + 1) >> 1;
    }
  }
  return v[0];
}

// ---- chunk loads and stores ---------------------------------------------------
// NT = true: non-temporal access, for data touched once by a layout in which
// each load or store instruction covers whole cache lines (consecutive lanes,
// consecutive addresses: SwiGLU, RoPE).  On such streams it measures 5-10%
// faster than a cached access; layouts that split a line over several
// instructions of one lane (the chunk-per-thread reductions) must stay
// cached, or every instruction refetches the line.
template <bool NT, typename V>
__device__ __forceinline__ V vload(const V *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename V>
__device__ __forceinline__ void vstore(V *p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// AL = false: element-wise accesses, for rows whose starts are not aligned
// to the vector width; the chunk (and so the tree) is the same either way.
template <int CH, bool NT = false, bool AL = true>
__device__ __forceinline__ void load_bf16(float (&v)[CH], const uint16_t *p) {
  if constexpr (!AL) {
#pragma unroll
    for (int e = 0; e < CH; ++e) v[e] = bf2f(p[e]);
  } else if constexpr (CH >= 8) {
#pragma unroll
    for (int q = 0; q < CH / 8; ++q) {
      const u32x4 u = vload<NT>(reinterpret_cast<const u32x4 *>(p + 8 * q));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * q + 2 * e] = __uint_as_float(u[e] << 16);
        v[8 * q + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
      }
    }
  } else if constexpr (CH == 4) {
    const u32x2 u = vload<NT>(reinterpret_cast<const u32x2 *>(p));
    v[0] = __uint_as_float(u[0] << 16); v[1] = __uint_as_float(u[0] & 0xffff0000u);
    v[2] = __uint_as_float(u[1] << 16); v[3] = __uint_as_float(u[1] & 0xffff0000u);
  } else {
#pragma unroll
    for (int e = 0; e < CH; ++e) v[e] = bf2f(p[e]);
  }
}

template <int CH, bool NT = false, bool AL = true>
__device__ __forceinline__ void store_bf16(uint16_t *p, const float (&v)[CH]) {
  if constexpr (!AL) {
#pragma unroll
    for (int e = 0; e < CH; ++e) p[e] = f2bf(v[e]);
  } else if constexpr (CH >= 8) {
#pragma unroll
    for (int q = 0; q < CH / 8; ++q) {
      u32x4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = pack_bf16(v[8 * q + 2 * e], v[8 * q + 2 * e + 1]);
      vstore<NT>(reinterpret_cast<u32x4 *>(p + 8 * q), u);
    }
  } else if constexpr (CH == 4) {
    u32x2 u;
    u[0] = pack_bf16(v[0], v[1]);
    u[1] = pack_bf16(v[2], v[3]);
    vstore<NT>(reinterpret_cast<u32x2 *>(p), u);
  } else {
#pragma unroll
    for (int e = 0; e < CH; ++e) p[e] = f2bf(v[e]);
  }
}

template <int CH, bool NT = false, bool AL = true>
__device__ __forceinline__ void load_f32(float (&v)[CH], const float *p) {
  if constexpr (AL && CH >= 4) {
#pragma unroll
    for (int q = 0; q < CH / 4; ++q) {
      const f32x4 u = vload<NT>(reinterpret_cast<const f32x4 *>(p + 4 * q));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = u[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < CH; ++e) v[e] = p[e];
  }
}

// Largest power of two <= 16 dividing G.
static int chunk_for(int64_t G) {
  int ch = 16;
  while (ch > 1 && (G % ch) != 0) ch >>= 1;
  return ch;
}

// Largest power of two <= 16 (in elements of `elem` bytes) that divides the
// element offset of p and the row stride ld: the alignment of every row start.
static int elem_align(const void *p, int64_t ld, int elem) {
  int a = 16;
  const uintptr_t off = (uintptr_t)p / (uintptr_t)elem;
  while (a > 1 && (((off % a) != 0) || (ld % a) != 0)) a >>= 1;
  if ((uintptr_t)p % elem) a = 1;
  return a;
}

// Element alignment that vector accesses of a CH-wide chunk need: 16-byte
// accesses for 8 or more bf16 (4 or more fp32), 8-byte for 4 bf16; narrower
// chunks are accessed element by element.  Rows aligned below that take the
// element-wise instance of the same kernel: the chunk width (and with it the
// tree, the LDS staging and the set of accepted shapes) depends only on the
// shape, never on alignment.
static bool bf16_vec_ok(int ch, int align) {
  return ch < 4 || align >= (ch >= 8 ? 8 : 4);
}
static bool f32_vec_ok(int ch, int align) { return ch < 4 || align >= 4; }

// =============================================================================
// residual-add + RMSNorm: one workgroup per row.
// =============================================================================
constexpr int kRowThreads = 256;

// EACH (the misaligned rounding location): h = bf16(x + r) before the norm
// and n = bf16(h * rstd) before the weight, as eager bf16 arithmetic does.
template <int CH, bool EACH, bool AL>
__global__ void __launch_bounds__(kRowThreads)
k_rmsnorm(const uint16_t *x, const uint16_t *r, const uint16_t *w, uint16_t *y, uint16_t *r_out,
          int H, int64_t ld, float eps, int T) {
  extern __shared__ float lds[];
  const int nch = H / CH;
  const int gc = nch / T;
  const int64_t base = (int64_t)blockIdx.x * ld;
  const uint16_t *xr = x + base;
  const uint16_t *rr = r + base;
  for (int ch = threadIdx.x; ch < nch; ch += kRowThreads) {
    float a[CH], b[CH], sq[CH];
    load_bf16<CH, false, AL>(a, xr + ch * CH);
    load_bf16<CH, false, AL>(b, rr + ch * CH);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      a[e] = a[e] + b[e];          // h
      if (EACH) a[e] = bf_round(a[e]);
      sq[e] = a[e] * a[e];
    }
    if (r_out) store_bf16<CH, false, AL>(r_out + base + ch * CH, a);
    lds[ch] = chunk_tree<CH>(sq);
  }
  __syncthreads();
  const float ss = lds_row_tree<kRowThreads>(lds, lds + nch, gc, T);
  const float mean = ss / (float)H;
  const float rstd = 1.0f / __builtin_sqrtf(mean + eps);
  for (int ch = threadIdx.x; ch < nch; ch += kRowThreads) {
    float a[CH], b[CH], ww[CH];
    load_bf16<CH, false, AL>(a, xr + ch * CH);
    load_bf16<CH, false, AL>(b, rr + ch * CH);
    load_bf16<CH, false, AL>(ww, w + ch * CH);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      float h = a[e] + b[e];
      if (EACH) h = bf_round(h);
      float n = h * rstd;
      if (EACH) n = bf_round(n);
      a[e] = n * ww[e];
    }
    store_bf16<CH, false, AL>(y + base + ch * CH, a);
  }
}

// Register-resident variant: every thread owns at most one chunk, so h
// stays in registers between the sum of squares and the output (x and r are
// read once).  The chunks of one tree group are gc = G/CH consecutive
// threads, gc a power of two dividing 64, so PAIR over the group's chunk sums
// is a perfect tree evaluated as a butterfly over those lanes (xor 1, 2, 4,
// ...; every lane ends with the same bits since IEEE addition commutes).
// The T group sums meet in LDS for the top perfect tree.
template <int CH, bool EACH>
__global__ void __launch_bounds__(kRowThreads)
k_rmsnorm_reg(const uint16_t *x, const uint16_t *r, const uint16_t *w, uint16_t *y,
              uint16_t *r_out, int H, int64_t ld, float eps, int T, int gc) {
  __shared__ float gsum[8];
  const int nch = H / CH;
  const int ch = threadIdx.x;
  const bool own = ch < nch;
  const int64_t off = (int64_t)blockIdx.x * ld + (int64_t)ch * CH;
  float h[CH], ww[CH];
  float part = 0.0f;
  if (own) {
    float b[CH], sq[CH];
    load_bf16<CH>(h, x + off);
    load_bf16<CH>(b, r + off);
    load_bf16<CH>(ww, w + ch * CH);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      h[e] = h[e] + b[e];
      if (EACH) h[e] = bf_round(h[e]);
      sq[e] = h[e] * h[e];
    }
    if (r_out) store_bf16<CH>(r_out + off, h);
    part = chunk_tree<CH>(sq);
  }
  for (int o = 1; o < gc; o <<= 1) part = part + __shfl_xor(part, o);
  if (own && (ch & (gc - 1)) == 0) gsum[ch / gc] = part;
  __syncthreads();
  float g[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) g[q] = q < T ? gsum[q] : 0.0f;
  for (int wdt = T; wdt > 1; wdt >>= 1)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < wdt / 2) g[q] = g[2 * q] + g[2 * q + 1];
  const float mean = g[0] / (float)H;
  const float rstd = 1.0f / __builtin_sqrtf(mean + eps);
  if (own) {
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      float n = h[e] * rstd;
      if (EACH) n = bf_round(n);
      h[e] = n * ww[e];
    }
    store_bf16<CH>(y + off, h);
  }
}

// Rows of H = 2048 * U elements (U = 1, 2: groups of at most 32 chunks) in
// 16-element chunks: a chunk is read by two
// adjacent lanes (8 elements, 16 bytes each), so every load and store
// instruction of a wave covers 1 KB contiguously (non-temporal accesses
// measured slower here: TBIK_RMS_NT).  A lane reduces its half chunk (the chunk
// tree's level of 8), one lane-swap add finishes the chunk's perfect tree
// (the two lanes get the same bits: addition is commutative), and a
// butterfly over lane offsets 2, 4, .., gc evaluates each group's PAIR -- a
// perfect tree, gc being a power of two -- every lane of the group ending
// with the same bits.  Then as k_rmsnorm_reg.
#ifndef TBIK_RMS_PAIR
#define TBIK_RMS_PAIR 1
#endif
#ifndef TBIK_RMS_NT
#define TBIK_RMS_NT 0
#endif
template <int U, bool EACH>
__global__ void __launch_bounds__(kRowThreads)
k_rmsnorm_pair(const uint16_t *x, const uint16_t *r, const uint16_t *w, uint16_t *y,
               uint16_t *r_out, int H, int64_t ld, float eps, int T, int gc) {
  constexpr bool NT = TBIK_RMS_NT != 0;
  __shared__ float gsum[8];
  const int t = threadIdx.x, lane = t & 63;
  const int64_t rowoff = (int64_t)blockIdx.x * ld;
  float h[U][8], ww[U][8];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int unit = k * kRowThreads + t;          // elements 8*unit .. 8*unit+7
    float b[8], sq[8];
    load_bf16<8, NT>(h[k], x + rowoff + 8 * unit);
    load_bf16<8, NT>(b, r + rowoff + 8 * unit);
    load_bf16<8>(ww[k], w + 8 * unit);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[k][e] = h[k][e] + b[e];
      if (EACH) h[k][e] = bf_round(h[k][e]);
      sq[e] = h[k][e] * h[k][e];
    }
    if (r_out) store_bf16<8, NT>(r_out + rowoff + 8 * unit, h[k]);
    float part = chunk_tree<8>(sq);
    part = part + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                      0, __builtin_bit_cast(int, part), 0xB1, 0xf, 0xf, false));
    for (int o = 1; o < gc; o <<= 1) part = part + __shfl_xor(part, 2 * o);
    if ((lane & (2 * gc - 1)) == 0) gsum[(unit >> 1) / gc] = part;
  }
  __syncthreads();
  float g[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) g[q] = q < T ? gsum[q] : 0.0f;
  for (int wdt = T; wdt > 1; wdt >>= 1)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < wdt / 2) g[q] = g[2 * q] + g[2 * q + 1];
  const float mean = g[0] / (float)H;
  const float rstd = 1.0f / __builtin_sqrtf(mean + eps);
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int unit = k * kRowThreads + t;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float n = h[k][e] * rstd;
      if (EACH) n = bf_round(n);
      h[k][e] = n * ww[k][e];
    }
    store_bf16<8, NT>(y + rowoff + 8 * unit, h[k]);
  }
}

// Rows whose group size has too few factors of two for whole-group chunks
// (H / c > 8192 chunk sums): the sum of squares over 16-leaf chunks plus one
// tail item per group (TailRows), element-wise accesses; the output pass is
// element by element.
template <bool EACH>
__global__ void __launch_bounds__(kRowThreads)
k_rmsnorm_tail(const uint16_t *x, const uint16_t *r, const uint16_t *w, uint16_t *y,
               uint16_t *r_out, int H, int64_t ld, float eps, int T) {
  extern __shared__ float lds[];
  const TailRows L(H, T);
  const int n_it = T * L.gs;
  const int64_t base = (int64_t)blockIdx.x * ld;
  for (int it = threadIdx.x; it < n_it; it += kRowThreads) {
    int start, len;
    L.item(it, start, len);
    float sq[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sq[e] = 0.0f;
      if (e < len) {
        float h = bf2f(x[base + start + e]) + bf2f(r[base + start + e]);
        if (EACH) h = bf_round(h);
        if (r_out) r_out[base + start + e] = f2bf(h);
        sq[e] = h * h;
      }
    }
    lds[it] = pair16(sq, len);
  }
  __syncthreads();
  const float ss = lds_row_tree<kRowThreads>(lds, lds + n_it, L.gs, T);
  const float rstd = 1.0f / __builtin_sqrtf(ss / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += kRowThreads) {
    float h = bf2f(x[base + i]) + bf2f(r[base + i]);
    if (EACH) h = bf_round(h);
    float n = h * rstd;
    if (EACH) n = bf_round(n);
    y[base + i] = f2bf(n * bf2f(w[i]));
  }
}

template <bool EACH>
static int launch_rmsnorm_t(const uint16_t *x, const uint16_t *r, const uint16_t *w,
                            uint16_t *y, uint16_t *r_out, int rows, int H, int64_t ld,
                            float eps, hipStream_t s) {
  const int T = tree_T(H);
  int al = elem_align(x, ld, 2);
  al = al < elem_align(r, ld, 2) ? al : elem_align(r, ld, 2);
  al = al < elem_align(y, ld, 2) ? al : elem_align(y, ld, 2);
  al = al < elem_align(w, 16, 2) ? al : elem_align(w, 16, 2);
  if (r_out) al = al < elem_align(r_out, ld, 2) ? al : elem_align(r_out, ld, 2);
  const int ch = chunk_for(H / T);
  const bool vec = bf16_vec_ok(ch, al);
  const int nch = H / ch;
  dim3 grid((unsigned)rows), block(kRowThreads);
  if (nch > 8192) {
    // chunk sums and their ping-pong copy within 64 KB of LDS
    const int n_it = T * ((H / T) / 16 + ((H / T) % 16 ? 1 : 0));
    if (n_it > 8192) return TBIK_ERR_SHAPE;
    hipLaunchKernelGGL((k_rmsnorm_tail<EACH>), grid, block, 2 * (size_t)n_it * sizeof(float), s, x,
                       r, w, y, r_out, H, ld, eps, T);
    return check_launch();
  }
  const int gc = nch / T;
  if (vec && TBIK_RMS_PAIR && ch == 16 && H % (8 * kRowThreads) == 0 && (gc & (gc - 1)) == 0 &&
      gc <= 32) {
    switch (H / (8 * kRowThreads)) {
      case 1: hipLaunchKernelGGL((k_rmsnorm_pair<1, EACH>), grid, block, 0, s, x, r, w, y, r_out, H, ld, eps, T, gc); return check_launch();
      case 2: hipLaunchKernelGGL((k_rmsnorm_pair<2, EACH>), grid, block, 0, s, x, r, w, y, r_out, H, ld, eps, T, gc); return check_launch();
      default: break;
    }
  }
  if (vec && nch <= kRowThreads && (gc & (gc - 1)) == 0 && 64 % gc == 0) {
    switch (ch) {
      case 16: hipLaunchKernelGGL((k_rmsnorm_reg<16, EACH>), grid, block, 0, s, x, r, w, y, r_out, H, ld, eps, T, gc); break;
      case 8: hipLaunchKernelGGL((k_rmsnorm_reg<8, EACH>), grid, block, 0, s, x, r, w, y, r_out, H, ld, eps, T, gc); break;
      case 4: hipLaunchKernelGGL((k_rmsnorm_reg<4, EACH>), grid, block, 0, s, x, r, w, y, r_out, H, ld, eps, T, gc); break;
      case 2: hipLaunchKernelGGL((k_rmsnorm_reg<2, EACH>), grid, block, 0, s, x, r, w, y, r_out, H, ld, eps, T, gc); break;
      default: hipLaunchKernelGGL((k_rmsnorm_reg<1, EACH>), grid, block, 0, s, x, r, w, y, r_out, H, ld, eps, T, gc); break;
    }
    return check_launch();
  }
  const size_t lds = 2 * (size_t)nch * sizeof(float);
  switch (ch * 2 + (vec ? 1 : 0)) {
#define TBIK_RMS_CASE(CW, VEC)                                                                      \
  case CW * 2 + VEC:                                                                                \
    hipLaunchKernelGGL((k_rmsnorm<CW, EACH, VEC != 0>), grid, block, lds, s, x, r, w, y, r_out, H, \
                       ld, eps, T);                                                              \
    break;
    TBIK_RMS_CASE(16, 1) TBIK_RMS_CASE(16, 0) TBIK_RMS_CASE(8, 1) TBIK_RMS_CASE(8, 0)
    TBIK_RMS_CASE(4, 1) TBIK_RMS_CASE(4, 0) TBIK_RMS_CASE(2, 1) TBIK_RMS_CASE(1, 1)
#undef TBIK_RMS_CASE
    default: return TBIK_ERR_SHAPE;
  }
  return check_launch();
}

int launch_rmsnorm_residual(const uint16_t *x, const uint16_t *r, const uint16_t *w,
                            uint16_t *y, uint16_t *r_out, int rows, int H, int64_t ld,
                            float eps, int rounding, hipStream_t s) {
  return rounding == TBIK_ROUND_EACH_OP
             ? launch_rmsnorm_t<true>(x, r, w, y, r_out, rows, H, ld, eps, s)
             : launch_rmsnorm_t<false>(x, r, w, y, r_out, rows, H, ld, eps, s);
}

#ifndef TBIK_ROPE_HPT
#define TBIK_ROPE_HPT 2
#endif
// =============================================================================
// RoPE (rotate-half).  One thread = 4 consecutive pairs (i..i+3, i+h..i+h+3);
// grid.x covers the (head, pair-quad) items of one token, grid.y the tokens.
// =============================================================================
// EACH: table entries and every product rounded to bf16 before the
// difference and the sum (rotate_half arithmetic on bf16 tensors).
// INV: the rotation by -angle, the adjoint used by the backward pass:
// y[i] = x[i]*c + x[i+h]*s, y[i+h] = x[i+h]*c - x[i]*s.
// HPT: heads per thread.  With HPT > 1 a thread rotates the same 4 pairs of
// HPT heads (heads hg, hg + heads/HPT, ...), so one load of the token's
// table entries serves all of them; the lanes of one instruction still read
// whole 128-byte half rows.
template <bool EACH, bool INV = false, int HPT = 1>
__global__ void __launch_bounds__(256)
k_rope(const uint16_t *x, uint16_t *y, const int32_t *pos, const float *cos_tab,
       const float *sin_tab, int T, int heads, int half, int64_t ld_token, int max_pos,
       int q4_shift) {
  const int q4 = half / 4;                       // 4-pair items per head
  const int hstride = heads / HPT;
  const int item = blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= hstride * q4) return;
  const int hd0 = q4_shift >= 0 ? item >> q4_shift : item / q4;
  const int i = (item - hd0 * q4) * 4;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    int p = pos[t];
    p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
    f32x4 c = *reinterpret_cast<const f32x4 *>(cos_tab + (int64_t)p * half + i);
    f32x4 sn = *reinterpret_cast<const f32x4 *>(sin_tab + (int64_t)p * half + i);
    if constexpr (EACH) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = bf_round(c[e]);
        sn[e] = bf_round(sn[e]);
      }
    }
    u32x2 ua[HPT], ub[HPT];
#pragma unroll
    for (int k = 0; k < HPT; ++k) {
      const int64_t off = (int64_t)t * ld_token + (int64_t)(hd0 + k * hstride) * 2 * half + i;
      ua[k] = vload<true>(reinterpret_cast<const u32x2 *>(x + off));
      ub[k] = vload<true>(reinterpret_cast<const u32x2 *>(x + off + half));
    }
#pragma unroll
    for (int k = 0; k < HPT; ++k) {
    const int64_t off = (int64_t)t * ld_token + (int64_t)(hd0 + k * hstride) * 2 * half + i;
    const float a[4] = {__uint_as_float(ua[k][0] << 16), __uint_as_float(ua[k][0] & 0xffff0000u),
                        __uint_as_float(ua[k][1] << 16), __uint_as_float(ua[k][1] & 0xffff0000u)};
    const float b[4] = {__uint_as_float(ub[k][0] << 16), __uint_as_float(ub[k][0] & 0xffff0000u),
                        __uint_as_float(ub[k][1] << 16), __uint_as_float(ub[k][1] & 0xffff0000u)};
    float ya[4], yb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float ac = a[e] * c[e], bs = b[e] * sn[e];
      float bc = b[e] * c[e], as = a[e] * sn[e];
      if constexpr (EACH) {
        ac = bf_round(ac);
        bs = bf_round(bs);
        bc = bf_round(bc);
        as = bf_round(as);
      }
      ya[e] = INV ? ac + bs : ac - bs;
      yb[e] = INV ? bc - as : bc + as;
    }
    u32x2 oa, ob;
    oa[0] = pack_bf16(ya[0], ya[1]);
    oa[1] = pack_bf16(ya[2], ya[3]);
    ob[0] = pack_bf16(yb[0], yb[1]);
    ob[1] = pack_bf16(yb[2], yb[3]);
    vstore<true>(reinterpret_cast<u32x2 *>(y + off), oa);
    vstore<true>(reinterpret_cast<u32x2 *>(y + off + half), ob);
    }
  }
}

int launch_rope(const uint16_t *x, uint16_t *y, const int32_t *pos, const float *cos_tab,
                const float *sin_tab, int T, int heads, int head_dim, int64_t ld_token,
                int max_pos, int rounding, hipStream_t s) {
  if (T == 0) return TBIK_OK;
  const int half = head_dim / 2;
  const int q4 = half / 4;
  int q4_shift = -1;
  for (int b = 0; b < 31; ++b)
    if ((1 << b) == q4) q4_shift = b;
  const unsigned gy = (unsigned)(T < 65535 ? T : 65535);
  if (TBIK_ROPE_HPT > 1 && heads % TBIK_ROPE_HPT == 0) {
    const int ipt = heads / TBIK_ROPE_HPT * q4;          // items per token
    const int bs = ipt >= 256 ? 256 : (ipt + 63) / 64 * 64;
    const unsigned gx = (unsigned)((ipt + bs - 1) / bs);
    if (rounding == kRopeInverse)
      hipLaunchKernelGGL((k_rope<false, true, TBIK_ROPE_HPT>), dim3(gx, gy), dim3(bs), 0, s, x, y,
                         pos, cos_tab, sin_tab, T, heads, half, ld_token, max_pos, q4_shift);
    else if (rounding == TBIK_ROUND_EACH_OP)
      hipLaunchKernelGGL((k_rope<true, false, TBIK_ROPE_HPT>), dim3(gx, gy), dim3(bs), 0, s, x, y,
                         pos, cos_tab, sin_tab, T, heads, half, ld_token, max_pos, q4_shift);
    else
      hipLaunchKernelGGL((k_rope<false, false, TBIK_ROPE_HPT>), dim3(gx, gy), dim3(bs), 0, s, x, y,
                         pos, cos_tab, sin_tab, T, heads, half, ld_token, max_pos, q4_shift);
    return check_launch();
  }
  const int items = heads * q4;
  const unsigned gx = (unsigned)((items + 255) / 256);
  if (rounding == kRopeInverse)
    hipLaunchKernelGGL((k_rope<false, true>), dim3(gx, gy), dim3(256), 0, s, x, y, pos, cos_tab,
                       sin_tab, T, heads, half, ld_token, max_pos, q4_shift);
  else if (rounding == TBIK_ROUND_EACH_OP)
    hipLaunchKernelGGL((k_rope<true>), dim3(gx, gy), dim3(256), 0, s, x, y, pos, cos_tab, sin_tab, T,
                       heads, half, ld_token, max_pos, q4_shift);
  else
    hipLaunchKernelGGL((k_rope<false>), dim3(gx, gy), dim3(256), 0, s, x, y, pos, cos_tab, sin_tab, T,
                       heads, half, ld_token, max_pos, q4_shift);
  return check_launch();
}

// =============================================================================
// SwiGLU: out = bf16((g / (1 + EXP(-g))) * u).  8 elements per item.
// =============================================================================
// silu, silu_n: tbik_device.h (shared with the GEMM's fused SwiGLU epilogue).

// grid.x covers the 8-element items of a row, grid.y the rows.
// EACH: the activation is rounded to bf16 before the product with u.
template <bool VEC, bool EACH>
__global__ void __launch_bounds__(256)
k_swiglu(const uint16_t *g, const uint16_t *u, uint16_t *o, int rows, int cols, int64_t ldg,
         int64_t ldu, int64_t ldo) {
  const int per = VEC ? 8 : 1;
  const int col = (blockIdx.x * blockDim.x + threadIdx.x) * per;
  if (col >= cols) return;
  for (int row = blockIdx.y; row < rows; row += gridDim.y) {
    if constexpr (VEC) {
      float gv[8], uv[8];
      load_bf16<8, true>(gv, g + (int64_t)row * ldg + col);
      load_bf16<8, true>(uv, u + (int64_t)row * ldu + col);
      silu_n<8>(gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) gv[e] = (EACH ? bf_round(gv[e]) : gv[e]) * uv[e];
      store_bf16<8, true>(o + (int64_t)row * ldo + col, gv);
    } else {
      float a = silu(bf2f(g[(int64_t)row * ldg + col]));
      if (EACH) a = bf_round(a);
      o[(int64_t)row * ldo + col] = f2bf(a * bf2f(u[(int64_t)row * ldu + col]));
    }
  }
}

int launch_swiglu(const uint16_t *g, const uint16_t *u, uint16_t *o, int rows, int cols,
                  int64_t ldg, int64_t ldu, int64_t ldo, int rounding, hipStream_t s) {
  if (rows == 0 || cols == 0) return TBIK_OK;
  const bool vec = (cols % 8) == 0 && elem_align(g, ldg, 2) >= 8 && elem_align(u, ldu, 2) >= 8 &&
                   elem_align(o, ldo, 2) >= 8;
  const int items = vec ? cols / 8 : cols;
  const dim3 grid((unsigned)((items + 255) / 256), (unsigned)(rows < 65535 ? rows : 65535));
  const bool each = rounding == TBIK_ROUND_EACH_OP;
  if (vec && each)
    hipLaunchKernelGGL((k_swiglu<true, true>), grid, dim3(256), 0, s, g, u, o, rows, cols, ldg, ldu, ldo);
  else if (vec)
    hipLaunchKernelGGL((k_swiglu<true, false>), grid, dim3(256), 0, s, g, u, o, rows, cols, ldg, ldu, ldo);
  else if (each)
    hipLaunchKernelGGL((k_swiglu<false, true>), grid, dim3(256), 0, s, g, u, o, rows, cols, ldg, ldu, ldo);
  else
    hipLaunchKernelGGL((k_swiglu<false, false>), grid, dim3(256), 0, s, g, u, o, rows, cols, ldg, ldu, ldo);
  return check_launch();
}

// =============================================================================
// log-softmax + gather: one workgroup per row, one kernel.
//  pass 1: m = exact row maximum (fmax; order-free);
//  pass 2: e = EXP(x - m) per leaf, chunk trees -> LDS (reverse chunk order,
//          so the first re-reads hit the lines pass 1 fetched last);
//  PAIR levels of every group in place in LDS (node i of a level sits at
//  i * 2^level, so the carried odd element never moves), then the shard
//  nodes (perfect trees over T/tp groups), their perfect tree, LOG, gather.
// =============================================================================
#ifndef TBIK_LSM_THREADS
#define TBIK_LSM_THREADS 1024
#endif
#ifndef TBIK_LSM_LDS_MIN
#define TBIK_LSM_LDS_MIN 0
#endif
constexpr int kLsmThreads = TBIK_LSM_THREADS;
// 16-element chunks read by lane quads (1 = on), with non-temporal loads
// (NT; a plus only with whole-line accesses) and KB loads in flight per lane
#ifndef TBIK_LSM_QUAD
#define TBIK_LSM_QUAD 1
#endif
#ifndef TBIK_LSM_NT
#define TBIK_LSM_NT 1
#endif
#ifndef TBIK_LSM_KB
#define TBIK_LSM_KB 8
#endif

// PAIR over each of `groups` groups of m values, group g at buf[g*m ..), in
// place, level by level (node i of a level sits at i * 2^level, so the
// carried odd element never moves); the group's PAIR value is left at
// buf[g*m].  groups is a power of two dividing NT: each group gets NT/groups
// threads (no division in the index arithmetic).  All threads of the block
// call it; every level ends with a block barrier.
template <int NT>
__device__ __forceinline__ void lds_pair_inplace(float *buf, int m, int groups) {
  const int sh = __builtin_ctz((unsigned)(NT / groups));
  float *gb = buf + (threadIdx.x >> sh) * m;
  const int r = threadIdx.x & ((1 << sh) - 1);
  int s = 1;
  while (m > 1) {
    const int half = m >> 1;
    for (int i = r; i < half; i += 1 << sh) {
      float *b = gb + 2 * i * s;
      b[0] = b[0] + b[s];
    }
    __syncthreads();
    s <<= 1;
    m = half + (m & 1);
  }
}

// The last steps of a row, by one thread: the group PAIR values (lds[g*gs]
// after lds_pair_inplace) form the tp shard nodes by the perfect
// tree over T/tp groups each, the nodes their perfect tree; then LOG and the
// target's logprob.  The caller has read the target index tgt and its logit
// xt (any value when tgt is out of range) before the row's sum, so that
// neither read waits at the end of the row.
__device__ __forceinline__ void lsm_finish(const float *lds, int gs, int T, int tp, int row,
                                           float *shard, float *out, float xt, float m, int tgt,
                                           int V) {
  const int per = T / tp;
  float nodes[8];
  for (int t = 0; t < tp; ++t) {
    float u[8];
    for (int q = 0; q < per; ++q) u[q] = lds[(t * per + q) * gs];
    for (int w = per; w > 1; w >>= 1)
      for (int q = 0; q < w / 2; ++q) u[q] = u[2 * q] + u[2 * q + 1];
    nodes[t] = u[0];
    shard[(int64_t)row * tp + t] = u[0];
  }
  for (int w = tp; w > 1; w >>= 1)
    for (int q = 0; q < w / 2; ++q) nodes[q] = nodes[2 * q] + nodes[2 * q + 1];
  if (tgt < 0 || tgt >= V) {
    out[row] = __builtin_nanf("");
    return;
  }
  out[row] = (xt - m) - log_f32(nodes[0]);
}

// The target's logit, for thread 0 (the one that finishes the row).
__device__ __forceinline__ float lsm_target_logit(const float *xr, int tgt, int V) {
  return (threadIdx.x == 0 && tgt >= 0 && tgt < V) ? xr[tgt] : 0.0f;
}

// This thread's share of a row's partial maxima: four loads in flight per
// round (one round up to 4 x kLsmThreads values).
__device__ __forceinline__ float lsm_pmax_part(const float *pm, int npmax) {
  float m = -__builtin_inff();
  for (int b0 = threadIdx.x; b0 < npmax; b0 += 4 * kLsmThreads) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = b0 + i * kLsmThreads;
      v[i] = b < npmax ? pm[b] : -__builtin_inff();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) m = __builtin_fmaxf(m, v[i]);
  }
  return m;
}

// Row maximum (order-free): from partial maxima when given, else from the
// logits element by element.  Every thread returns the row's maximum.
__device__ __forceinline__ float lsm_row_max(const float *xr, int V, const float *pmax,
                                             int64_t ld_pmax, int npmax, int row, float *red) {
  float m = -__builtin_inff();
  if (pmax) {
    m = lsm_pmax_part(pmax + (int64_t)row * ld_pmax, npmax);
  } else {
    for (int i = threadIdx.x; i < V; i += kLsmThreads) m = __builtin_fmaxf(m, xr[i]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int q = 1; q < kLsmThreads / 64; ++q) m = __builtin_fmaxf(m, red[q]);
  return m;
}

// Rows whose group size has too few factors of two for whole-group chunks to
// fit LDS (G = V / T odd, say): 16-leaf chunks plus one tail item per group
// (TailRows), element-wise loads (group starts need not be aligned); the
// maximum and the rest of the row as in the main kernel.
__global__ void __launch_bounds__(kLsmThreads)
k_logsoftmax_row_tail(const float *logits, int64_t ld, const int32_t *targets, int V, int T,
                      int tp, float *shard, float *out, const float *pmax, int64_t ld_pmax,
                      int npmax) {
  extern __shared__ float lds[];
  __shared__ float red[kLsmThreads / 64];
  const int row = blockIdx.x;
  const float *xr = logits + (int64_t)row * ld;
  const TailRows L(V, T);
  const int tgt = threadIdx.x == 0 ? targets[row] : 0;
  const float m = lsm_row_max(xr, V, pmax, ld_pmax, npmax, row, red);
  const float xt = lsm_target_logit(xr, tgt, V);
  for (int it = threadIdx.x; it < T * L.gs; it += kLsmThreads) {
    int start, len;
    L.item(it, start, len);
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = e < len ? exp_f32(xr[start + e] - m) : 0.0f;
    lds[it] = pair16(v, len);
  }
  __syncthreads();
  lds_pair_inplace<kLsmThreads>(lds, L.gs, T);
  if (threadIdx.x == 0) lsm_finish(lds, L.gs, T, tp, row, shard, out, xt, m, tgt, V);
}

template <int CH, bool AL>
__global__ void __launch_bounds__(kLsmThreads)
k_logsoftmax_row(const float *logits, int64_t ld, const int32_t *targets, int V, int T, int tp,
                 float *shard, float *out, const float *pmax, int64_t ld_pmax, int npmax) {
  extern __shared__ float lds[];
  __shared__ float red[kLsmThreads / 64];
  const int row = blockIdx.x;
  const float *xr = logits + (int64_t)row * ld;
  const int nch = V / CH;
  const int gc = nch / T;
  const int tgt = threadIdx.x == 0 ? targets[row] : 0;
  // Quad path (16-element chunks, aligned rows).  A chunk is read by a quad
  // of lanes, lane j of the quad holding its elements 4j..4j+3, so every load
  // instruction of a wave covers 1 KB contiguously.  Each lane reduces its
  // four values (the chunk tree's level of 4), and two quad-permute adds
  // finish the chunk's perfect tree: (q0 + q1) + (q2 + q3) -- addition is
  // commutative, so every lane of the quad ends with the same bits.
  // A unit is 16 chunks (1 KB, one load of a wave).  Wave w takes units w,
  // w + NWV, w + 2 NWV, ... counted from the row's end, so the waves' shares
  // differ by at most one unit, KB units per step.  Buffer loads from a
  // resource of the row's size: a partial last unit reads zeros past the
  // row (those chunks are not stored); in a wave's last step the units past
  // its share get an offset beyond the resource, which reads nothing, so
  // that every step issues its KB loads together.  Non-temporal loads: the row is read once
  // here when its maximum comes from the GEMM.  The first step's loads go
  // out before the row maximum is formed (they do not depend on it).
  constexpr bool QUAD = AL && CH == 16 && TBIK_LSM_QUAD;
  constexpr int NWV = kLsmThreads / 64;
  constexpr int KB = TBIK_LSM_KB;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // wave-uniform
  const int qd = lane >> 2, j = lane & 3;
  const int nunit = (nch + 15) / 16;
  const int cnt = wv < nunit ? (nunit - 1 - wv) / NWV + 1 : 0;
  f32x4 ua[KB];
  __amdgpu_buffer_rsrc_t rs;
  // the chunk index of step i0's k-th unit for this lane
  auto chunk = [&](int i0, int k) { return (nunit - 1 - wv - NWV * (i0 + k)) * 16 + qd; };
  auto issue = [&](f32x4 (&u)[KB], int i0) {
    const int n = cnt - i0 < KB ? cnt - i0 : KB;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int off = k < n ? chunk(i0, k) * 64 + 16 * j : 0x40000000;
      u[k] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, TBIK_LSM_NT ? 2 : 0));
    }
  };
  if constexpr (QUAD) {
    rs = __builtin_amdgcn_make_buffer_rsrc((void *)xr, (short)0, nch * 64, 0x00020000);
    issue(ua, 0);
  }
  float m = -__builtin_inff();
  if (pmax) {
    // the row maximum from partial maxima (e.g. fused into the GEMM that
    // produced the logits): the logits are then read once
    m = lsm_pmax_part(pmax + (int64_t)row * ld_pmax, npmax);
  } else if constexpr (AL && CH >= 4) {
    // the maximum is order-free: consecutive lanes read consecutive 16 bytes
    for (int i = threadIdx.x; i < nch * (CH / 4); i += kLsmThreads) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + 4 * i);
      m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3])));
    }
  } else {
    for (int ch = threadIdx.x; ch < nch; ch += kLsmThreads) {
      float v[CH];
      load_f32<CH, false, AL>(v, xr + ch * CH);
#pragma unroll
      for (int e = 0; e < CH; ++e) m = __builtin_fmaxf(m, v[e]);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int q = 1; q < kLsmThreads / 64; ++q) m = __builtin_fmaxf(m, red[q]);
  const float xt = lsm_target_logit(xr, tgt, V);
  if constexpr (QUAD) {
    // EXP's NaN case is taken once per lane's four values: a NaN argument
    // makes the chunk's sum NaN whichever element it was, and the clamped
    // main path is harmless for NaN (it gives a finite value that the select
    // then replaces).  Other values take exactly exp_f32's main path.
    auto consume = [&](const f32x4 (&u)[KB], int i0) {
      const int n = cnt - i0 < KB ? cnt - i0 : KB;
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        if (k >= n) break;
        float e[4];
        bool nan = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = u[k][i] - m;
          nan = nan || (d != d);
          e[i] = exp_core(exp_clamp(d));
        }
        float t = (e[0] + e[1]) + (e[2] + e[3]);
        if (nan) t = __builtin_nanf("");
        t = t + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                    0, __builtin_bit_cast(int, t), 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
        t = t + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                    0, __builtin_bit_cast(int, t), 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
        const int c = chunk(i0, k);
        if (j == 0 && c < nch) lds[c] = t;
      }
    };
    for (int i0 = 0;;) {
      consume(ua, i0);
      i0 += KB;
      if (i0 >= cnt) break;
      issue(ua, i0);
    }
  } else {
    for (int ch = nch - 1 - (int)threadIdx.x; ch >= 0; ch -= kLsmThreads) {
      float v[CH];
      load_f32<CH, false, AL>(v, xr + ch * CH);
#pragma unroll
      for (int e = 0; e < CH; ++e) v[e] = exp_f32(v[e] - m);
      lds[ch] = chunk_tree<CH>(v);
    }
  }
  __syncthreads();
  lds_pair_inplace<kLsmThreads>(lds, gc, T);
  if (threadIdx.x == 0) lsm_finish(lds, gc, T, tp, row, shard, out, xt, m, tgt, V);
}

int launch_logsoftmax(const float *logits, int64_t ld, const int32_t *targets, float *out, int M,
                      int V, int tp, float *ws, const float *pmax, int64_t ld_pmax, int npmax,
                      hipStream_t s) {
  if (M == 0) return TBIK_OK;
  const int T = tree_T(V);
  const int G = V / T;
  const int ch = chunk_for(G);
  const bool vec = f32_vec_ok(ch, elem_align(logits, ld, 4));
  const int nch = V / ch;
  size_t lds = (size_t)nch * sizeof(float);
  // one float per chunk in dynamic LDS, beside the kernel's static per-wave
  // reduction buffer, within a workgroup's 160 KB
  constexpr size_t kLdsCap = 160 * 1024 - (size_t)(kLsmThreads / 64) * sizeof(float);
  if (lds > kLdsCap) {
    // G with few factors of two: 16-leaf chunks plus one tail value per group
    const size_t lt = (size_t)T * (G / 16 + (G % 16 ? 1 : 0)) * sizeof(float);
    if (lt > kLdsCap) return TBIK_ERR_SHAPE;
    (void)hipFuncSetAttribute((const void *)k_logsoftmax_row_tail,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lt);
    hipLaunchKernelGGL(k_logsoftmax_row_tail, dim3((unsigned)M), dim3(kLsmThreads), lt, s, logits,
                       ld, targets, V, T, tp, ws, out, pmax, ld_pmax, npmax);
    return check_launch();
  }
  if (lds < (size_t)TBIK_LSM_LDS_MIN) lds = TBIK_LSM_LDS_MIN;
  float *shard = ws;
  dim3 grid((unsigned)M), block(kLsmThreads);
  switch (ch * 2 + (vec ? 1 : 0)) {
#define TBIK_LSM_CASE(CW, VEC)                                                                    \
  case CW * 2 + VEC:                                                                              \
    if (lds > 64 * 1024)                                                                       \
      (void)hipFuncSetAttribute((const void *)k_logsoftmax_row<CW, VEC != 0>,                     \
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);               \
    hipLaunchKernelGGL((k_logsoftmax_row<CW, VEC != 0>), grid, block, lds, s, logits, ld, targets, \
                       V, T, tp, shard, out, pmax, ld_pmax, npmax);                            \
    break;
    TBIK_LSM_CASE(16, 1) TBIK_LSM_CASE(16, 0) TBIK_LSM_CASE(8, 1) TBIK_LSM_CASE(8, 0)
    TBIK_LSM_CASE(4, 1) TBIK_LSM_CASE(4, 0) TBIK_LSM_CASE(2, 1) TBIK_LSM_CASE(1, 1)
#undef TBIK_LSM_CASE
    default: return TBIK_ERR_SHAPE;
  }
  return check_launch();
}

// =============================================================================
// causal softmax: one workgroup per (batch, query row).
// =============================================================================
// Rows whose group size has too few factors of two for whole-group chunks
// (Lk / c > 8192 chunk sums): 16-leaf chunks plus one tail item per group
// (TailRows), element-wise accesses; otherwise as k_softmax_causal.
__global__ void __launch_bounds__(kRowThreads)
k_softmax_causal_tail(const float *S, int64_t ld_s, int64_t stride_s, uint16_t *P, int64_t ld_p,
                      int64_t stride_p, int Lq, int Lk, int offset, float scale, int T) {
  extern __shared__ float lds[];
  __shared__ float red[kRowThreads / 64];
  const int i = blockIdx.x, b = blockIdx.y;
  const float *srow = S + (int64_t)b * stride_s + (int64_t)i * ld_s;
  uint16_t *prow = P + (int64_t)b * stride_p + (int64_t)i * ld_p;
  const int last = i + offset;
  const TailRows L(Lk, T);
  const int n_it = T * L.gs;
  float m = -__builtin_inff();
  for (int k = threadIdx.x; k < Lk; k += kRowThreads)
    if (k <= last) m = __builtin_fmaxf(m, srow[k] * scale);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int q = 1; q < kRowThreads / 64; ++q) m = __builtin_fmaxf(m, red[q]);
  for (int it = threadIdx.x; it < n_it; it += kRowThreads) {
    int start, len;
    L.item(it, start, len);
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
      v[e] = (e < len && start + e <= last) ? exp_f32(srow[start + e] * scale - m) : 0.0f;
    lds[it] = pair16(v, len);
  }
  __syncthreads();
  const float ssum = lds_row_tree<kRowThreads>(lds, lds + n_it, L.gs, T);
  for (int k = threadIdx.x; k < Lk; k += kRowThreads)
    prow[k] = f2bf(k <= last ? exp_f32(srow[k] * scale - m) / ssum : 0.0f);
}

template <int CH, bool AL>
__global__ void __launch_bounds__(kRowThreads)
k_softmax_causal(const float *S, int64_t ld_s, int64_t stride_s, uint16_t *P, int64_t ld_p,
                 int64_t stride_p, int Lq, int Lk, int offset, float scale, int T) {
  extern __shared__ float lds[];
  __shared__ float red[kRowThreads / 64];
  const int i = blockIdx.x, b = blockIdx.y;
  const float *srow = S + (int64_t)b * stride_s + (int64_t)i * ld_s;
  uint16_t *prow = P + (int64_t)b * stride_p + (int64_t)i * ld_p;
  const int last = i + offset;
  const int nch = Lk / CH;
  const int gc = nch / T;
  float m = -__builtin_inff();
  for (int ch = threadIdx.x; ch < nch; ch += kRowThreads) {
    float v[CH];
    load_f32<CH, false, AL>(v, srow + ch * CH);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const float z = v[e] * scale;
      if (ch * CH + e <= last) m = __builtin_fmaxf(m, z);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int q = 1; q < kRowThreads / 64; ++q) m = __builtin_fmaxf(m, red[q]);
  for (int ch = threadIdx.x; ch < nch; ch += kRowThreads) {
    float v[CH];
    load_f32<CH, false, AL>(v, srow + ch * CH);
#pragma unroll
    for (int e = 0; e < CH; ++e) v[e] = (ch * CH + e <= last) ? exp_f32(v[e] * scale - m) : 0.0f;
    lds[ch] = chunk_tree<CH>(v);
  }
  __syncthreads();
  const float ssum = lds_row_tree<kRowThreads>(lds, lds + nch, gc, T);
  for (int ch = threadIdx.x; ch < nch; ch += kRowThreads) {
    float v[CH];
    load_f32<CH, false, AL>(v, srow + ch * CH);
#pragma unroll
    for (int e = 0; e < CH; ++e)
      v[e] = (ch * CH + e <= last) ? exp_f32(v[e] * scale - m) / ssum : 0.0f;
    store_bf16<CH, false, AL>(prow + ch * CH, v);
  }
}

// One wave per query row for Lk = 64 * CH (CH a power of two <= 16): lane l
// owns keys [l*CH, l*CH + CH).  Then T = 8, each group is 64/8 lanes and
// every level of the tree (chunk, PAIR of the group -- a perfect tree since
// the group size is a power of two -- and the top) is a perfect tree: the
// chunk tree in registers followed by a butterfly over all 64 lanes gives
// the row sum in every lane, with no LDS and no barrier.
template <int CH>
__global__ void __launch_bounds__(256)
k_softmax_causal_wave(const float *S, int64_t ld_s, int64_t stride_s, uint16_t *P, int64_t ld_p,
                      int64_t stride_p, int Lq, int offset, float scale) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (i >= Lq) return;
  const float *srow = S + (int64_t)b * stride_s + (int64_t)i * ld_s + lane * CH;
  uint16_t *prow = P + (int64_t)b * stride_p + (int64_t)i * ld_p + lane * CH;
  const int last = i + offset;
  float v[CH];
  load_f32<CH>(v, srow);
  float m = -__builtin_inff();
#pragma unroll
  for (int e = 0; e < CH; ++e) {
    v[e] = v[e] * scale;
    if (lane * CH + e <= last) m = __builtin_fmaxf(m, v[e]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  float ex[CH];
#pragma unroll
  for (int e = 0; e < CH; ++e) ex[e] = (lane * CH + e <= last) ? exp_f32(v[e] - m) : 0.0f;
  float t[CH];
#pragma unroll
  for (int e = 0; e < CH; ++e) t[e] = ex[e];
  float ssum = chunk_tree<CH>(t);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) ssum = ssum + __shfl_xor(ssum, off);
#pragma unroll
  for (int e = 0; e < CH; ++e) ex[e] = (lane * CH + e <= last) ? ex[e] / ssum : 0.0f;
  store_bf16<CH>(prow, ex);
}

int launch_softmax_causal(const float *S, int64_t ld_s, int64_t stride_s, uint16_t *P,
                          int64_t ld_p, int64_t stride_p, int Lq, int Lk, int batch, int offset,
                          float scale, hipStream_t s) {
  const int T = tree_T(Lk);
  {
    // one wave per row when Lk = 64 * CH and every row start allows the
    // vector accesses of a CH-wide chunk
    const int chw = Lk / 64;
    const int as = elem_align(S, ld_s, 4) < elem_align(S, stride_s, 4) ? elem_align(S, ld_s, 4)
                                                                       : elem_align(S, stride_s, 4);
    const int ap = elem_align(P, ld_p, 2) < elem_align(P, stride_p, 2) ? elem_align(P, ld_p, 2)
                                                                       : elem_align(P, stride_p, 2);
    if (Lk % 64 == 0 && (chw & (chw - 1)) == 0 && chw <= 16 && as >= (chw < 4 ? chw : 4) &&
        ap >= (chw < 8 ? chw : 8)) {
      dim3 g((unsigned)((Lq + 3) / 4), (unsigned)batch), blk(256);
      switch (chw) {
        case 16: hipLaunchKernelGGL(k_softmax_causal_wave<16>, g, blk, 0, s, S, ld_s, stride_s, P, ld_p, stride_p, Lq, offset, scale); break;
        case 8: hipLaunchKernelGGL(k_softmax_causal_wave<8>, g, blk, 0, s, S, ld_s, stride_s, P, ld_p, stride_p, Lq, offset, scale); break;
        case 4: hipLaunchKernelGGL(k_softmax_causal_wave<4>, g, blk, 0, s, S, ld_s, stride_s, P, ld_p, stride_p, Lq, offset, scale); break;
        case 2: hipLaunchKernelGGL(k_softmax_causal_wave<2>, g, blk, 0, s, S, ld_s, stride_s, P, ld_p, stride_p, Lq, offset, scale); break;
        default: hipLaunchKernelGGL(k_softmax_causal_wave<1>, g, blk, 0, s, S, ld_s, stride_s, P, ld_p, stride_p, Lq, offset, scale); break;
      }
      return check_launch();
    }
  }
  int ch = chunk_for(Lk / T);
  if (ch > 8) ch = 8;
  const int as = elem_align(S, ld_s, 4) < elem_align(S, stride_s, 4) ? elem_align(S, ld_s, 4)
                                                                     : elem_align(S, stride_s, 4);
  const int ap = elem_align(P, ld_p, 2) < elem_align(P, stride_p, 2) ? elem_align(P, ld_p, 2)
                                                                     : elem_align(P, stride_p, 2);
  const bool vec = f32_vec_ok(ch, as) && bf16_vec_ok(ch, ap);
  const int nch = Lk / ch;
  const size_t lds = 2 * (size_t)nch * sizeof(float);
  dim3 grid((unsigned)Lq, (unsigned)batch), block(kRowThreads);
  if (nch > 8192) {
    const int n_it = T * ((Lk / T) / 16 + ((Lk / T) % 16 ? 1 : 0));
    if (n_it > 8192) return TBIK_ERR_SHAPE;
    hipLaunchKernelGGL(k_softmax_causal_tail, grid, block, 2 * (size_t)n_it * sizeof(float), s, S,
                       ld_s, stride_s, P, ld_p, stride_p, Lq, Lk, offset, scale, T);
    return check_launch();
  }
  switch (ch * 2 + (vec ? 1 : 0)) {
#define TBIK_SMC_CASE(CW, VEC)                                                                    \
  case CW * 2 + VEC:                                                                              \
    hipLaunchKernelGGL((k_softmax_causal<CW, VEC != 0>), grid, block, lds, s, S, ld_s, stride_s, P, \
                       ld_p, stride_p, Lq, Lk, offset, scale, T);                              \
    break;
    TBIK_SMC_CASE(8, 1) TBIK_SMC_CASE(8, 0) TBIK_SMC_CASE(4, 1) TBIK_SMC_CASE(4, 0)
    TBIK_SMC_CASE(2, 1) TBIK_SMC_CASE(1, 1)
#undef TBIK_SMC_CASE
    default: return TBIK_ERR_SHAPE;
  }
  return check_launch();
}

// =============================================================================
// row gather (embedding lookup): out[i] = table[idx[i]], zero row when the
// index is out of range.  grid.x covers the columns, grid.y the rows.
// =============================================================================
template <bool VEC>
__global__ void __launch_bounds__(256)
k_gather_rows(const uint16_t *table, int64_t ld_table, int rows, const int32_t *idx, int n,
              int cols, uint16_t *out, int64_t ld_out) {
  const int per = VEC ? 8 : 1;
  const int col = (blockIdx.x * blockDim.x + threadIdx.x) * per;
  if (col >= cols) return;
  for (int i = blockIdx.y; i < n; i += gridDim.y) {
    const int r = idx[i];
    const bool ok = r >= 0 && r < rows;
    if constexpr (VEC) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4 *>(table + (int64_t)r * ld_table + col);
      vstore<true>(reinterpret_cast<u32x4 *>(out + (int64_t)i * ld_out + col), v);
    } else {
      out[(int64_t)i * ld_out + col] = ok ? table[(int64_t)r * ld_table + col] : (uint16_t)0;
    }
  }
}

int launch_gather_rows(const uint16_t *table, int64_t ld_table, int rows, const int32_t *idx,
                       int n, int cols, uint16_t *out, int64_t ld_out, hipStream_t s) {
  if (n == 0 || cols == 0) return TBIK_OK;
  const bool vec = (cols % 8) == 0 && elem_align(table, ld_table, 2) >= 8 &&
                   elem_align(out, ld_out, 2) >= 8;
  const int items = vec ? cols / 8 : cols;
  const dim3 grid((unsigned)((items + 255) / 256), (unsigned)(n < 65535 ? n : 65535));
  if (vec)
    hipLaunchKernelGGL(k_gather_rows<true>, grid, dim3(256), 0, s, table, ld_table, rows, idx, n,
                       cols, out, ld_out);
  else
    hipLaunchKernelGGL(k_gather_rows<false>, grid, dim3(256), 0, s, table, ld_table, rows, idx, n,
                       cols, out, ld_out);
  return check_launch();
}

// =============================================================================
// primitives, elementwise
// =============================================================================
__global__ void __launch_bounds__(256) k_primitive(int op, const float *x, float *y, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = x[i];
    float r;
    if (op == TBIK_PRIM_EXP) r = exp_f32(v);
    else if (op == TBIK_PRIM_LOG) r = log_f32(v);
    else if (op == TBIK_PRIM_BF16) r = bf2f(f2bf(v));
    else r = silu(bf2f(f2bf(v)));
    y[i] = r;
  }
}

int launch_primitive(int op, const float *x, float *y, int64_t n, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 262144) blocks = 262144;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_primitive, dim3((unsigned)blocks), dim3(256), 0, s, op, x, y, n);
  return check_launch();
}

// =============================================================================
// Backward passes (training side).  fp32 intermediates in the order the
// header gives, each output rounded once to bf16; sums over tokens are trees
// over 64-token leaves whose T groups are the data-parallel shards.
// =============================================================================
int launch_rope_backward(const uint16_t *dy, uint16_t *dx, const int32_t *pos,
                         const float *cos_tab, const float *sin_tab, int T, int heads,
                         int head_dim, int64_t ld_token, int max_pos, hipStream_t s) {
  return launch_rope(dy, dx, pos, cos_tab, sin_tab, T, heads, head_dim, ld_token, max_pos,
                     kRopeInverse, s);
}

// SwiGLU backward: du = bf16(d * silu(g)),
// dg = bf16((d * u) * (sig * (1 + g * (1 - sig)))) with sig = 1 / (1 + EXP(-g))
// and silu = g / (1 + EXP(-g)), both divisions correctly rounded.
__device__ __forceinline__ void swiglu_bwd_1(float g, float u, float d, float &dg, float &du) {
  const float den = silu_den(g);
  const float sig = 1.0f / den;
  const float sl = g / den;
  du = d * sl;
  dg = (d * u) * (sig * (1.0f + g * (1.0f - sig)));
}

template <bool VEC>
__global__ void __launch_bounds__(256)
k_swiglu_bwd(const uint16_t *g, const uint16_t *u, const uint16_t *d, uint16_t *dg, uint16_t *du,
             int rows, int cols, int64_t ldg, int64_t ldu, int64_t ldd, int64_t lddg,
             int64_t lddu) {
  const int per = VEC ? 8 : 1;
  const int col = (blockIdx.x * blockDim.x + threadIdx.x) * per;
  if (col >= cols) return;
  for (int row = blockIdx.y; row < rows; row += gridDim.y) {
    if constexpr (VEC) {
      float gv[8], uv[8], dv[8], og[8], ou[8];
      load_bf16<8, true>(gv, g + (int64_t)row * ldg + col);
      load_bf16<8, true>(uv, u + (int64_t)row * ldu + col);
      load_bf16<8, true>(dv, d + (int64_t)row * ldd + col);
#pragma unroll
      for (int e = 0; e < 8; ++e) swiglu_bwd_1(gv[e], uv[e], dv[e], og[e], ou[e]);
      store_bf16<8, true>(dg + (int64_t)row * lddg + col, og);
      store_bf16<8, true>(du + (int64_t)row * lddu + col, ou);
    } else {
      float og, ou;
      swiglu_bwd_1(bf2f(g[(int64_t)row * ldg + col]), bf2f(u[(int64_t)row * ldu + col]),
                   bf2f(d[(int64_t)row * ldd + col]), og, ou);
      dg[(int64_t)row * lddg + col] = f2bf(og);
      du[(int64_t)row * lddu + col] = f2bf(ou);
    }
  }
}

int launch_swiglu_backward(const uint16_t *g, const uint16_t *u, const uint16_t *d, uint16_t *dg,
                           uint16_t *du, int rows, int cols, int64_t ldg, int64_t ldu,
                           int64_t ldd, int64_t lddg, int64_t lddu, hipStream_t s) {
  if (rows == 0 || cols == 0) return TBIK_OK;
  const bool vec = (cols % 8) == 0 && elem_align(g, ldg, 2) >= 8 && elem_align(u, ldu, 2) >= 8 &&
                   elem_align(d, ldd, 2) >= 8 && elem_align(dg, lddg, 2) >= 8 &&
                   elem_align(du, lddu, 2) >= 8;
  const int items = vec ? cols / 8 : cols;
  const dim3 grid((unsigned)((items + 255) / 256), (unsigned)(rows < 65535 ? rows : 65535));
  if (vec)
    hipLaunchKernelGGL(k_swiglu_bwd<true>, grid, dim3(256), 0, s, g, u, d, dg, du, rows, cols,
                       ldg, ldu, ldd, lddg, lddu);
  else
    hipLaunchKernelGGL(k_swiglu_bwd<false>, grid, dim3(256), 0, s, g, u, d, dg, du, rows, cols,
                       ldg, ldu, ldd, lddg, lddu);
  return check_launch();
}

// Residual RMSNorm backward, one workgroup per row: rstd from the forward's
// tree (same chunks, same LDS tree, same bits), dot = TREE(g*h) with
// g = dy*w, c = (dot * ((rstd*rstd)*rstd)) / H, dh = bf16(((rstd*g) - (c*h)) + dr).
// rstd of the row goes to rstd_out for the weight gradient.
// Rows whose group size has too few factors of two for whole-group chunks
// (H / c > 8192 chunk sums): both row trees over 16-leaf chunks plus one tail
// item per group (TailRows), element-wise accesses; otherwise as
// k_rmsnorm_bwd.
__global__ void __launch_bounds__(kRowThreads)
k_rmsnorm_bwd_tail(const uint16_t *x, const uint16_t *r, const uint16_t *w, const uint16_t *dy,
                   const uint16_t *dr, uint16_t *dh, float *rstd_out, int H, int64_t ld,
                   float eps, int T) {
  extern __shared__ float lds[];
  const TailRows L(H, T);
  const int n_it = T * L.gs;
  const int64_t base = (int64_t)blockIdx.x * ld;
  for (int it = threadIdx.x; it < n_it; it += kRowThreads) {
    int start, len;
    L.item(it, start, len);
    float a[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      a[e] = 0.0f;
      if (e < len) {
        const float h = bf2f(x[base + start + e]) + bf2f(r[base + start + e]);
        a[e] = h * h;
      }
    }
    lds[it] = pair16(a, len);
  }
  __syncthreads();
  const float ss = lds_row_tree<kRowThreads>(lds, lds + n_it, L.gs, T);
  const float rstd = 1.0f / __builtin_sqrtf(ss / (float)H + eps);
  __syncthreads();                       // every thread has read the root
  for (int it = threadIdx.x; it < n_it; it += kRowThreads) {
    int start, len;
    L.item(it, start, len);
    float a[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      a[e] = 0.0f;
      if (e < len) {
        const int64_t o = base + start + e;
        a[e] = (bf2f(dy[o]) * bf2f(w[start + e])) * (bf2f(x[o]) + bf2f(r[o]));
      }
    }
    lds[it] = pair16(a, len);
  }
  __syncthreads();
  const float dot = lds_row_tree<kRowThreads>(lds, lds + n_it, L.gs, T);
  const float c = (dot * ((rstd * rstd) * rstd)) / (float)H;
  for (int k = threadIdx.x; k < H; k += kRowThreads) {
    const int64_t o = base + k;
    const float h = bf2f(x[o]) + bf2f(r[o]);
    float v = (rstd * (bf2f(dy[o]) * bf2f(w[k]))) - (c * h);
    if (dr) v = v + bf2f(dr[o]);
    dh[o] = f2bf(v);
  }
  if (threadIdx.x == 0) rstd_out[blockIdx.x] = rstd;
}

template <int CH, bool AL>
__global__ void __launch_bounds__(kRowThreads)
k_rmsnorm_bwd(const uint16_t *x, const uint16_t *r, const uint16_t *w, const uint16_t *dy,
              const uint16_t *dr, uint16_t *dh, float *rstd_out, int H, int64_t ld, float eps,
              int T) {
  extern __shared__ float lds[];
  const int nch = H / CH;
  const int gc = nch / T;
  const int64_t base = (int64_t)blockIdx.x * ld;
  for (int ch = threadIdx.x; ch < nch; ch += kRowThreads) {
    float a[CH], b[CH];
    load_bf16<CH, false, AL>(a, x + base + ch * CH);
    load_bf16<CH, false, AL>(b, r + base + ch * CH);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      a[e] = a[e] + b[e];
      a[e] = a[e] * a[e];
    }
    lds[ch] = chunk_tree<CH>(a);
  }
  __syncthreads();
  const float ss = lds_row_tree<kRowThreads>(lds, lds + nch, gc, T);
  const float rstd = 1.0f / __builtin_sqrtf(ss / (float)H + eps);
  __syncthreads();                       // every thread has read the root
  for (int ch = threadIdx.x; ch < nch; ch += kRowThreads) {
    float a[CH], b[CH], gy[CH], ww[CH];
    load_bf16<CH, false, AL>(a, x + base + ch * CH);
    load_bf16<CH, false, AL>(b, r + base + ch * CH);
    load_bf16<CH, false, AL>(gy, dy + base + ch * CH);
    load_bf16<CH, false, AL>(ww, w + ch * CH);
#pragma unroll
    for (int e = 0; e < CH; ++e) a[e] = (gy[e] * ww[e]) * (a[e] + b[e]);
    lds[ch] = chunk_tree<CH>(a);
  }
  __syncthreads();
  const float dot = lds_row_tree<kRowThreads>(lds, lds + nch, gc, T);
  const float c = (dot * ((rstd * rstd) * rstd)) / (float)H;
  for (int ch = threadIdx.x; ch < nch; ch += kRowThreads) {
    float a[CH], b[CH], gy[CH], ww[CH], gr[CH];
    load_bf16<CH, false, AL>(a, x + base + ch * CH);
    load_bf16<CH, false, AL>(b, r + base + ch * CH);
    load_bf16<CH, false, AL>(gy, dy + base + ch * CH);
    load_bf16<CH, false, AL>(ww, w + ch * CH);
    if (dr) load_bf16<CH, false, AL>(gr, dr + base + ch * CH);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const float h = a[e] + b[e];
      float v = (rstd * (gy[e] * ww[e])) - (c * h);
      if (dr) v = v + gr[e];
      a[e] = v;
    }
    store_bf16<CH, false, AL>(dh + base + ch * CH, a);
  }
  if (threadIdx.x == 0) rstd_out[blockIdx.x] = rstd;
}

// Register-resident variant (the forward's k_rmsnorm_reg layout and tree):
// every thread owns at most one chunk, x/r/dy/w/dr are read once; the two
// row trees are the chunk tree, a butterfly over the gc lanes of a group
// (a perfect tree, gc a power of two dividing 64) and the perfect top over
// the T group sums in LDS.
template <int CH>
__global__ void __launch_bounds__(kRowThreads)
k_rmsnorm_bwd_reg(const uint16_t *x, const uint16_t *r, const uint16_t *w, const uint16_t *dy,
                  const uint16_t *dr, uint16_t *dh, float *rstd_out, int H, int64_t ld, float eps,
                  int T, int gc) {
  __shared__ float gsum[2][8];
  const int nch = H / CH;
  const int ch = threadIdx.x;
  const bool own = ch < nch;
  const int64_t off = (int64_t)blockIdx.x * ld + (int64_t)ch * CH;
  float h[CH], g[CH];
  float part = 0.0f;
  if (own) {
    float b[CH], ww[CH], sq[CH];
    load_bf16<CH>(h, x + off);
    load_bf16<CH>(b, r + off);
    load_bf16<CH>(g, dy + off);
    load_bf16<CH>(ww, w + ch * CH);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      h[e] = h[e] + b[e];
      sq[e] = h[e] * h[e];
      g[e] = g[e] * ww[e];
    }
    part = chunk_tree<CH>(sq);
  }
  for (int o = 1; o < gc; o <<= 1) part = part + __shfl_xor(part, o);
  if (own && (ch & (gc - 1)) == 0) gsum[0][ch / gc] = part;
  float q2 = 0.0f;
  if (own) {
    float q[CH];
#pragma unroll
    for (int e = 0; e < CH; ++e) q[e] = g[e] * h[e];
    q2 = chunk_tree<CH>(q);
  }
  for (int o = 1; o < gc; o <<= 1) q2 = q2 + __shfl_xor(q2, o);
  if (own && (ch & (gc - 1)) == 0) gsum[1][ch / gc] = q2;
  __syncthreads();
  float t0[8], t1[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    t0[q] = q < T ? gsum[0][q] : 0.0f;
    t1[q] = q < T ? gsum[1][q] : 0.0f;
  }
  for (int wdt = T; wdt > 1; wdt >>= 1)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < wdt / 2) {
        t0[q] = t0[2 * q] + t0[2 * q + 1];
        t1[q] = t1[2 * q] + t1[2 * q + 1];
      }
  const float rstd = 1.0f / __builtin_sqrtf(t0[0] / (float)H + eps);
  const float c = (t1[0] * ((rstd * rstd) * rstd)) / (float)H;
  if (own) {
    float gr[CH];
    if (dr) load_bf16<CH>(gr, dr + off);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      float v = (rstd * g[e]) - (c * h[e]);
      if (dr) v = v + gr[e];
      h[e] = v;
    }
    store_bf16<CH>(dh + off, h);
  }
  if (threadIdx.x == 0) rstd_out[blockIdx.x] = rstd;
}

// Leaves of the weight gradient: leaf b of column j adds
// dy_ij * ((x_ij + r_ij) * rstd_i) over the 64 rows of leaf b in row order
// from +0.  grid.x covers the columns (one per thread), grid.y the leaves.
// VEC = 2: two consecutive columns per thread (4-byte loads; a leaf is a
// sequential sum, so the parallelism is columns x leaves), else one.
template <int VEC>
__global__ void __launch_bounds__(256)
k_rmsnorm_dw_leaves(const uint16_t *x, const uint16_t *r, const uint16_t *dy, const float *rstd,
                    float *leaves, int H, int64_t ld) {
  const int col = (blockIdx.x * blockDim.x + threadIdx.x) * VEC;
  if (col >= H) return;
  const int r0 = blockIdx.y * 64;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll 8
  for (int i = 0; i < 64; ++i) {
    const int64_t o = (int64_t)(r0 + i) * ld + col;
    const float rs = rstd[r0 + i];
    float a[VEC], b[VEC], gy[VEC];
    if constexpr (VEC == 2) {
      const uint32_t ua = *reinterpret_cast<const uint32_t *>(x + o);
      const uint32_t ub = *reinterpret_cast<const uint32_t *>(r + o);
      const uint32_t ug = *reinterpret_cast<const uint32_t *>(dy + o);
      a[0] = __uint_as_float(ua << 16); a[1] = __uint_as_float(ua & 0xffff0000u);
      b[0] = __uint_as_float(ub << 16); b[1] = __uint_as_float(ub & 0xffff0000u);
      gy[0] = __uint_as_float(ug << 16); gy[1] = __uint_as_float(ug & 0xffff0000u);
    } else {
      a[0] = bf2f(x[o]); b[0] = bf2f(r[o]); gy[0] = bf2f(dy[o]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = acc[e] + gy[e] * ((a[e] + b[e]) * rs);
  }
  float *out = leaves + (int64_t)blockIdx.y * H + col;
#pragma unroll
  for (int e = 0; e < VEC; ++e) out[e] = acc[e];
}

// Tree over the nleaf leaves of each column: PAIR inside each of the T
// groups, then the shards (perfect trees over T/dp groups; shard nodes to
// shards[dp][H] when not null) and the perfect tree over the dp shards.
// T/dp and dp are powers of two, so this is the perfect top over the T
// groups for every dp.
// Block (64, T): thread (c, q) evaluates PAIR over group q of column c;
// the group values meet in LDS and lane q == 0 finishes the column.
__global__ void __launch_bounds__(512)
k_colsum_tree(const float *leaves, int nleaf, int H, int T, int dp, float *shards, float *out) {
  __shared__ float gs[8][64];
  const int col = blockIdx.x * 64 + threadIdx.x;
  const int q = threadIdx.y;
  const int G = nleaf / T;
  if (col < H) {
    float st[20][1];
    float node[1] = {0.0f};
    // the leaves are requested 8 at a time (independent loads in flight),
    // then pushed in order
    for (int i0 = 0; i0 < G; i0 += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k < G ? i0 + k : G - 1;
        v[k] = leaves[(int64_t)(q * G + i) * H + col];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (i0 + k < G) {
          node[0] = v[k];
          pair_push<1, 20>(st, node, i0 + k, G);
        }
      }
    }
    gs[q][threadIdx.x] = node[0];
  }
  __syncthreads();
  if (q != 0 || col >= H) return;
  float gv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) gv[k] = k < T ? gs[k][threadIdx.x] : 0.0f;
  const int per = T / dp;
  float sv[8];
  for (int t = 0; t < dp; ++t) {
    float v[8];
    for (int k = 0; k < per; ++k) v[k] = gv[t * per + k];
    for (int wdt = per; wdt > 1; wdt >>= 1)
      for (int k = 0; k < wdt / 2; ++k) v[k] = v[2 * k] + v[2 * k + 1];
    sv[t] = v[0];
    if (shards) shards[(int64_t)t * H + col] = v[0];
  }
  for (int wdt = dp; wdt > 1; wdt >>= 1)
    for (int k = 0; k < wdt / 2; ++k) sv[k] = sv[2 * k] + sv[2 * k + 1];
  out[col] = sv[0];
}

int launch_rmsnorm_backward(const uint16_t *x, const uint16_t *r, const uint16_t *w,
                            const uint16_t *dy, const uint16_t *dr, uint16_t *dh, float *dw,
                            int rows, int H, int64_t ld, float eps, int dp, float *ws,
                            hipStream_t s) {
  const int T = tree_T(H);
  int al = elem_align(x, ld, 2);
  al = al < elem_align(r, ld, 2) ? al : elem_align(r, ld, 2);
  al = al < elem_align(dy, ld, 2) ? al : elem_align(dy, ld, 2);
  al = al < elem_align(dh, ld, 2) ? al : elem_align(dh, ld, 2);
  al = al < elem_align(w, 16, 2) ? al : elem_align(w, 16, 2);
  if (dr) al = al < elem_align(dr, ld, 2) ? al : elem_align(dr, ld, 2);
  const int ch = chunk_for(H / T);
  const bool vec = bf16_vec_ok(ch, al);
  const int nch = H / ch;
  const size_t lds = 2 * (size_t)nch * sizeof(float);
  float *rstd = ws;                                 // [rows]
  const dim3 grid((unsigned)rows), block(kRowThreads);
  const int gc = nch / T;
  if (nch > 8192) {
    const int n_it = T * ((H / T) / 16 + ((H / T) % 16 ? 1 : 0));
    if (n_it > 8192) return TBIK_ERR_SHAPE;
    hipLaunchKernelGGL(k_rmsnorm_bwd_tail, grid, block, 2 * (size_t)n_it * sizeof(float), s, x, r,
                       w, dy, dr, dh, rstd, H, ld, eps, T);
  } else if (vec && nch <= kRowThreads && (gc & (gc - 1)) == 0 && 64 % gc == 0) {
    switch (ch) {
      case 16: hipLaunchKernelGGL(k_rmsnorm_bwd_reg<16>, grid, block, 0, s, x, r, w, dy, dr, dh, rstd, H, ld, eps, T, gc); break;
      case 8: hipLaunchKernelGGL(k_rmsnorm_bwd_reg<8>, grid, block, 0, s, x, r, w, dy, dr, dh, rstd, H, ld, eps, T, gc); break;
      case 4: hipLaunchKernelGGL(k_rmsnorm_bwd_reg<4>, grid, block, 0, s, x, r, w, dy, dr, dh, rstd, H, ld, eps, T, gc); break;
      case 2: hipLaunchKernelGGL(k_rmsnorm_bwd_reg<2>, grid, block, 0, s, x, r, w, dy, dr, dh, rstd, H, ld, eps, T, gc); break;
      default: hipLaunchKernelGGL(k_rmsnorm_bwd_reg<1>, grid, block, 0, s, x, r, w, dy, dr, dh, rstd, H, ld, eps, T, gc); break;
    }
  } else switch (ch * 2 + (vec ? 1 : 0)) {
#define TBIK_RMSB_CASE(CW, VEC)                                                                   \
  case CW * 2 + VEC:                                                                              \
    hipLaunchKernelGGL((k_rmsnorm_bwd<CW, VEC != 0>), grid, block, lds, s, x, r, w, dy, dr, dh,     \
                       rstd, H, ld, eps, T);                                                   \
    break;
    TBIK_RMSB_CASE(16, 1) TBIK_RMSB_CASE(16, 0) TBIK_RMSB_CASE(8, 1) TBIK_RMSB_CASE(8, 0)
    TBIK_RMSB_CASE(4, 1) TBIK_RMSB_CASE(4, 0) TBIK_RMSB_CASE(2, 1) TBIK_RMSB_CASE(1, 1)
#undef TBIK_RMSB_CASE
    default: return TBIK_ERR_SHAPE;
  }
  int rc = check_launch();
  if (rc != TBIK_OK || !dw) return rc;
  const int nleaf = rows / 64;
  float *leaves = ws + rmsnorm_bwd_rstd_floats(rows);
  float *shards = leaves + (int64_t)nleaf * H;
  const bool pairs = (H % 2) == 0 && elem_align(x, ld, 2) >= 2 && elem_align(r, ld, 2) >= 2 &&
                     elem_align(dy, ld, 2) >= 2;
  if (pairs)
    hipLaunchKernelGGL(k_rmsnorm_dw_leaves<2>, dim3((unsigned)((H / 2 + 255) / 256), (unsigned)nleaf),
                       dim3(256), 0, s, x, r, dy, rstd, leaves, H, ld);
  else
    hipLaunchKernelGGL(k_rmsnorm_dw_leaves<1>, dim3((unsigned)((H + 255) / 256), (unsigned)nleaf),
                       dim3(256), 0, s, x, r, dy, rstd, leaves, H, ld);
  rc = check_launch();
  if (rc != TBIK_OK) return rc;
  const int Tl = tree_T(nleaf);
  hipLaunchKernelGGL(k_colsum_tree, dim3((unsigned)((H + 63) / 64)), dim3(64, (unsigned)Tl), 0, s,
                     leaves, nleaf, H, Tl, dp, shards, dw);
  return check_launch();
}

}  // namespace tbik
