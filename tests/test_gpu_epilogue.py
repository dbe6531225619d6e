"""The GEMM's output stores through the C ABI (fp32, bf16 and the SwiGLU
epilogue's H): the full-line path (fp32 or bf16 outputs with 16-byte aligned
rows: the tile staged in LDS and written as whole rows) and the direct path
(any other output) write exactly the outputs of a strided, offset output
view, bit for bit what a contiguous output receives, and nothing outside it
(the rest of the buffer holds NaN sentinels)."""
import pytest
import torch

import tp_invariant_numerics_amd as tb
from tp_invariant_numerics_amd import inputs

DEV = "cuda"
pytestmark = pytest.mark.gpu

# (M, N, K, element offset of C in its buffer, extra row pitch)
CASES = [(512, 4112, 4096, 0, 8),      # aligned rows: full-line path
         (300, 4111, 1024, 0, 9),      # aligned pitch, ragged N
         (257, 130, 2048, 1, 4),       # misaligned base: direct path
         (4096, 1000, 1024, 0, 0),     # contiguous, many row tiles
         (129, 4096, 14336, 3, 12),    # split K and the combine kernel, misaligned
         (64, 256, 64, 0, 4)]          # one leaf


def _strided(M, N, off, pad):
    ldc = N + pad
    buf = torch.full(((M + 2) * ldc + off + 64,), float("nan"), device=DEV)
    C = buf[off: off + M * ldc].view(M, ldc)[:, :N]
    mask = torch.ones(buf.shape, dtype=torch.bool, device=DEV)
    mask[off: off + M * ldc].view(M, ldc)[:, :N] = False
    return buf, C, mask


@pytest.mark.parametrize("M,N,K,off,pad", CASES)
def test_gemm_strided_output(M, N, K, off, pad):
    print("case", M, N, K, off, pad, flush=True)
    A = inputs.normal_bf16((M, K), 900 + M, device=DEV)
    W = inputs.normal_bf16((N, K), 901 + N, std=0.02, device=DEV)
    ref = tb.tbik_gemm(A, W)[0]
    buf, C, mask = _strided(M, N, off, pad)
    tb.tbik_gemm(A, W, out=C)
    torch.cuda.synchronize()
    assert torch.equal(C.contiguous().view(torch.int32), ref.view(torch.int32))
    assert bool(torch.isnan(buf[mask]).all()), "a store landed outside the output view"


@pytest.mark.parametrize("M,N,K,off,pad", [(512, 4112, 4096, 0, 8), (200, 1000, 2048, 0, 12),
                                           (77, 2050, 1024, 2, 4)])
def test_logits_strided_output(M, N, K, off, pad):
    print("case", M, N, K, off, pad, flush=True)
    A = inputs.normal_bf16((M, K), 700 + M, device=DEV)
    W = inputs.normal_bf16((N, K), 701 + N, std=0.02, device=DEV)
    ref, pref = tb.tbik_gemm_logits(A, W)
    buf, C, mask = _strided(M, N, off, pad)
    _, pm = tb.tbik_gemm_logits(A, W, out=C)
    torch.cuda.synchronize()
    assert torch.equal(C.contiguous().view(torch.int32), ref.view(torch.int32))
    assert torch.equal(pm.view(torch.int32), pref.view(torch.int32))
    assert bool(torch.isnan(buf[mask]).all()), "a store landed outside the output view"


@pytest.mark.parametrize("M,N,K,off,pad", [(512, 4112, 4096, 0, 8), (300, 4111, 1024, 0, 9),
                                           (257, 130, 2048, 1, 6), (4096, 2048, 2048, 0, 0),
                                           (129, 4096, 14336, 3, 16)])
def test_gemm_bf16_strided_output(M, N, K, off, pad):
    """bf16-only output (full-line path when rows are 16-byte aligned): the
    round-to-nearest-even of the fp32 result, in a strided, offset view."""
    print("case", M, N, K, off, pad, flush=True)
    A = inputs.normal_bf16((M, K), 500 + M, device=DEV)
    W = inputs.normal_bf16((N, K), 501 + N, std=0.02, device=DEV)
    ref = tb.tbik_gemm(A, W)[0].to(torch.bfloat16)
    ldc = N + pad
    buf = torch.full(((M + 2) * ldc + off + 64,), float("nan"), dtype=torch.bfloat16, device=DEV)
    Cb = buf[off: off + M * ldc].view(M, ldc)[:, :N]
    mask = torch.ones(buf.shape, dtype=torch.bool, device=DEV)
    mask[off: off + M * ldc].view(M, ldc)[:, :N] = False
    tb.tbik_gemm(A, W, out_bf16=Cb, want_fp32=False)
    torch.cuda.synchronize()
    assert torch.equal(Cb.contiguous().view(torch.int16), ref.view(torch.int16))
    assert bool(torch.isnan(buf[mask]).all()), "a store landed outside the output view"


@pytest.mark.parametrize("M,F,K,off,pad", [(512, 2816, 2048, 0, 8), (300, 1040, 1024, 0, 16),
                                           (257, 208, 2048, 3, 5), (4096, 1024, 1024, 0, 0)])
def test_gemm_swiglu_strided_output(M, F, K, off, pad):
    """The gate/up GEMM with the SwiGLU node in its epilogue, H written into a
    strided, offset view: bit for bit the composition GEMM -> bf16 gate and
    up -> SwiGLU."""
    print("case", M, F, K, off, pad, flush=True)
    A = inputs.normal_bf16((M, K), 300 + M, device=DEV)
    Wgu = inputs.normal_bf16((2 * F, K), 301 + F, std=0.02, device=DEV)
    g = tb.tbik_gemm(A, Wgu[:F], want_fp32=False, want_bf16=True)[1]
    u = tb.tbik_gemm(A, Wgu[F:], want_fp32=False, want_bf16=True)[1]
    ref = tb.tbik_swiglu(g, u)
    ldh = F + pad
    buf = torch.full(((M + 2) * ldh + off + 64,), float("nan"), dtype=torch.bfloat16, device=DEV)
    H = buf[off: off + M * ldh].view(M, ldh)[:, :F]
    mask = torch.ones(buf.shape, dtype=torch.bool, device=DEV)
    mask[off: off + M * ldh].view(M, ldh)[:, :F] = False
    tb.tbik_gemm_swiglu(A, Wgu, out=H)
    torch.cuda.synchronize()
    assert torch.equal(H.contiguous().view(torch.int16), ref.view(torch.int16))
    assert bool(torch.isnan(buf[mask]).all()), "a store landed outside the output view"
