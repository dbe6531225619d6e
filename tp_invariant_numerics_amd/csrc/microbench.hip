// microbench.hip -- attainable ceilings of the chip, measured by the library's
// own kernels so that every roofline fraction can be quoted against both the
// published peak and what this GPU actually sustains.
//
//   k_mfma_peak   independent chains of v_mfma_f32_16x16x32_bf16 (the GEMM
//                 leaf instruction) from registers: no memory traffic in the
//                 loop, so its rate is the matrix cores' sustained peak.
//   k_hbm_read    non-temporal 16-byte loads (eight in flight per thread)
//                 over a buffer much larger than the last-level cache, folded
//                 by xor (one 4-byte store per thread at the end).
//   k_hbm_copy    non-temporal 16-byte loads and stores (four per thread in
//                 flight), src -> dst.
//   k_copy_lds    the GEMM ring's operand copy alone: 8 waves move 32 KB
//                 stages with 16-byte-per-lane global->LDS buffer loads into a
//                 4-slot LDS ring, 3 stages ahead, one barrier per stage, no
//                 MFMAs.  Over a window small enough to stay in every XCD's
//                 L2 it measures the L2 -> LDS delivery rate the 128x128 GEMM
//                 tiles depend on; over larger windows, the last-level cache
//                 and HBM through the same path.
//
// Grids are sized by the caller; every access is bounds-checked against the
// byte count (a multiple of 16).
#include "tbik_device.h"
#include "tbik_internal.h"
#include "../../include/tbik.h"

namespace tbik {

// CH independent accumulators per wave; `iters` rounds of CH chained MFMAs.
template <int CH>
__global__ void __launch_bounds__(512) k_mfma_peak(const u32x4 *seed, float *out, int iters) {
  const int lane = threadIdx.x & 63;
  u32x4 a = seed[lane], b = seed[64 + lane];
  f32x4 acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = f32x4{(float)c, 0.0f, 0.0f, 0.0f};   // distinct chains
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CH; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc[c], 0,
                                                       0, 0);
  }
  f32x4 s = acc[0];
#pragma unroll
  for (int c = 1; c < CH; ++c) s = s + acc[c];
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  out[t] = s[0] + s[1] + s[2] + s[3];
}

// Each workgroup streams consecutive chunks of 256 * U 16-byte units, U loads
// in flight per thread, so that every wave instruction covers 1 KB.
template <int U>
__global__ void __launch_bounds__(256) k_hbm_read(const u32x4 *src, int64_t n16, unsigned *out) {
  const int64_t chunk = 256 * U;
  u32x4 x = {0u, 0u, 0u, 0u};
  for (int64_t base = (int64_t)blockIdx.x * chunk; base < n16; base += (int64_t)gridDim.x * chunk) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u];
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

template <int U>
__global__ void __launch_bounds__(256) k_hbm_copy(const u32x4 *src, u32x4 *dst, int64_t n16) {
  const int64_t chunk = 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * chunk; base < n16; base += (int64_t)gridDim.x * chunk) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

typedef void __attribute__((address_space(3))) *mb_lptr_t;

// One workgroup: `stages` stages of 32 KB (32 segments of 1 KB, four per
// wave) read from a window of `nst` stages, starting at stage 7*blockIdx.x
// and wrapping, so concurrent workgroups read different lines.  Stage st goes
// to ring slot st % 4; after a wave issues stage st+3 it waits for its own
// loads of stage st (vector-memory counter <= 12) and the workgroup meets at
// a barrier, exactly the GEMM ring's protocol.  The tail re-reads the last
// stage, as the GEMM's does.
__global__ void __launch_bounds__(512) k_copy_lds(const void *src, unsigned nst, int stages,
                                                  unsigned *out) {
  constexpr int S = 4, SLOT = 2048;              // 16-byte units per 32 KB slot
  __shared__ u32x4 ring[S * SLOT];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, (int)(nst * 32768u), 0x00020000);
  const unsigned st0 = (blockIdx.x * 7u) % nst;
  unsigned voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (unsigned)((wave + 8 * i) * 1024 + lane * 16);
  auto issue = [&](int st, int slot) {
    const int sc = st < stages ? st : stages - 1;
    const int soff = (int)(((st0 + (unsigned)sc) % nst) * 32768u);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (mb_lptr_t)(ring + slot * SLOT + (wave + 8 * i) * 64), 16, voff[i], soff, 0, 0);
  };
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s, s);
  for (int st = 0; st < stages; ++st) {
    issue(st + S - 1, (st + S - 1) % S);
    // vmcnt <= 12 (gfx9 encoding: vmcnt [3:0] and [15:14]; expcnt, lgkmcnt unconstrained)
    __builtin_amdgcn_s_waitcnt((12 & 15) | ((12 >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const u32x4 v = ring[((stages - 1) % S) * SLOT + threadIdx.x];
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = v[0] ^ v[1] ^ v[2] ^ v[3];
}

static int mb_check() { return hipGetLastError() == hipSuccess ? TBIK_OK : TBIK_ERR_LAUNCH; }

}  // namespace tbik

using namespace tbik;

extern "C" {

int64_t tbik_bench_mfma_flops(int blocks, int iters) {
  if (blocks < 1 || iters < 1) return 0;
  // 8 waves per block, 8 chains each, 2*16*16*32 flops per instruction
  return (int64_t)blocks * 8 * 8 * (int64_t)iters * 16384;
}

int tbik_bench_mfma(const void *seed, float *out, int blocks, int iters, void *stream) {
  if (!seed || !out) return TBIK_ERR_NULL;
  if (blocks < 1 || blocks > (1 << 20) || iters < 1) return TBIK_ERR_SHAPE;
  if (((uintptr_t)seed & 15) != 0) return TBIK_ERR_ALIGN;
  hipLaunchKernelGGL(k_mfma_peak<8>, dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream,
                     (const u32x4 *)seed, out, iters);
  return mb_check();
}

int tbik_bench_hbm_read(const void *buf, int64_t bytes, unsigned *out, int blocks, void *stream) {
  if (!buf || !out) return TBIK_ERR_NULL;
  if (bytes <= 0 || (bytes & 15) != 0 || blocks < 1 || blocks > (1 << 20)) return TBIK_ERR_SHAPE;
  if (((uintptr_t)buf & 15) != 0) return TBIK_ERR_ALIGN;
  hipLaunchKernelGGL(k_hbm_read<8>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4 *)buf, bytes / 16, out);
  return mb_check();
}

int tbik_bench_hbm_copy(const void *src, void *dst, int64_t bytes, int blocks, void *stream) {
  if (!src || !dst) return TBIK_ERR_NULL;
  if (bytes <= 0 || (bytes & 15) != 0 || blocks < 1 || blocks > (1 << 20)) return TBIK_ERR_SHAPE;
  if ((((uintptr_t)src | (uintptr_t)dst) & 15) != 0) return TBIK_ERR_ALIGN;
  hipLaunchKernelGGL(k_hbm_copy<4>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4 *)src, (u32x4 *)dst, bytes / 16);
  return mb_check();
}

int tbik_bench_copy_lds(const void *buf, int64_t window_bytes, int stages, unsigned *out,
                        int blocks, void *stream) {
  if (!buf || !out) return TBIK_ERR_NULL;
  if (window_bytes < 32768 || (window_bytes & 32767) != 0 || window_bytes > ((int64_t)1 << 31) - 32768 ||
      stages < 1 || blocks < 1 || blocks > (1 << 20))
    return TBIK_ERR_SHAPE;
  if (((uintptr_t)buf & 15) != 0) return TBIK_ERR_ALIGN;
  hipLaunchKernelGGL(k_copy_lds, dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream, buf,
                     (unsigned)(window_bytes / 32768), stages, out);
  return mb_check();
}

}  // extern "C"
