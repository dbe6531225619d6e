// training.hip -- operand layout for the training-side GEMMs.
//
// The backward GEMMs reduce over N (input gradient dX = dY W) and over the
// tokens M (weight gradient dW = dY^T X).  The tree GEMM kernels read both
// operands with the reduced dimension contiguous, so the gradients first
// transpose the operand(s) whose reduced dimension is strided: W for dX,
// dY and X for dW.  The transpose moves bits only, so the gradients keep
// the GEMM's tree (TREE over 64-wide leaves of the reduced dimension; TBIK
// summary page, "technical framework": one hierarchical binary tree for the
// reduction whatever the split), and a data-parallel split of the tokens is
// a split at aligned groups of that tree.
#include "tbik_device.h"
#include "tbik_internal.h"
#include "../../include/tbik.h"

namespace tbik {

namespace {

// y[c][r] = x[r][c] for one 64 x 64 tile per workgroup (256 threads).  The
// tile passes through LDS so that global reads and writes are both 16-byte
// row segments; the row pitch of 66 halves spreads a column read over all
// banks.  Edge tiles and unaligned layouts take element-wise paths.
constexpr int kTile = 64;
constexpr int kPitch = 66;

__global__ void __launch_bounds__(256)
k_transpose_bf16(const uint16_t *x, int64_t ldx, uint16_t *y, int64_t ldy, int rows, int cols,
                 int vec) {
  __shared__ uint16_t tile[kTile * kPitch];
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int t = threadIdx.x;
  const int seg = t & 7, rsub = t >> 3;          // 8 segments of 8 elements per row
  const bool full = vec && r0 + kTile <= rows && c0 + kTile <= cols;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = rsub + 32 * i;
    uint16_t v[8];
    if (full) {
      const u32x4 u = *reinterpret_cast<const u32x4 *>(x + (int64_t)(r0 + rr) * ldx + c0 + 8 * seg);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = (uint16_t)(u[e] & 0xffffu);
        v[2 * e + 1] = (uint16_t)(u[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = r0 + rr, c = c0 + 8 * seg + e;
        v[e] = (r < rows && c < cols) ? x[(int64_t)r * ldx + c] : (uint16_t)0;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[rr * kPitch + 8 * seg + e] = v[e];
  }
  __syncthreads();
  const bool full_out = vec && c0 + kTile <= cols && r0 + kTile <= rows;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int oc = rsub + 32 * i;                // output row = input column c0 + oc
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[(8 * seg + e) * kPitch + oc];
    if (full_out) {
      u32x4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = (uint32_t)v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
      *reinterpret_cast<u32x4 *>(y + (int64_t)(c0 + oc) * ldy + r0 + 8 * seg) = u;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int orow = c0 + oc, ocol = r0 + 8 * seg + e;
        if (orow < cols && ocol < rows) y[(int64_t)orow * ldy + ocol] = v[e];
      }
    }
  }
}

}  // namespace

int launch_transpose_bf16(const uint16_t *x, int64_t ldx, uint16_t *y, int64_t ldy, int rows,
                          int cols, hipStream_t s) {
  if (rows == 0 || cols == 0) return TBIK_OK;
  const int vec = (((uintptr_t)x | (uintptr_t)y) & 15u) == 0 && (ldx % 8) == 0 && (ldy % 8) == 0;
  const dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)((rows + kTile - 1) / kTile));
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, s, x, ldx, y, ldy, rows, cols, vec);
  return hipGetLastError() == hipSuccess ? TBIK_OK : TBIK_ERR_LAUNCH;
}

}  // namespace tbik
