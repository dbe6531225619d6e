"""GPU parity of the training-side calls (through the C ABI) against the oracle.

Bit-exact: the transpose, the scalar-leaf gradient GEMMs, and the RoPE,
SwiGLU and residual-RMSNorm backward passes (the RMSNorm weight gradient
with its token-axis tree for every simulated data-parallel split).  The
MFMA-leaf gradient GEMMs are held to the same bar as the forward GEMM:
bitwise invariance across the data-parallel split (TBIK summary page,
Abstract), exact integer results and a normwise error against binary64.
"""
import numpy as np
import pytest
import torch

import tp_invariant_numerics_amd as tb
from tp_invariant_numerics_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def bits(t):
    return inputs.bits(t)


def u32(a):
    return np.ascontiguousarray(np.asarray(a, np.float32)).view(np.uint32)


@pytest.mark.parametrize("rows,cols,pad", [(64, 64, 0), (130, 77, 0), (4096, 2048, 0),
                                           (100, 200, 8), (1, 9, 3)])
def test_transpose_bitexact(rows, cols, pad):
    x = inputs.normal_bf16((rows, cols + pad), 10000 + rows).to(DEV)[:, :cols]
    say("transpose", rows, cols, pad)
    y = tb.tbik_transpose_bf16(x)
    assert torch.equal(y.view(torch.int16), x.t().contiguous().view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(64, 128, 96), (33, 256, 200)])
def test_gemm_dgrad_scalar_bitexact(orc, M, N, K):
    dY = inputs.normal_bf16((M, N), 10100 + M)
    W = inputs.normal_bf16((N, K), 10101 + M, std=0.02)
    say("dgrad scalar", M, N, K)
    dX, dXb = tb.tbik_gemm_dgrad(dY.to(DEV), W.to(DEV), leaf_mode=tb.LEAF_SCALAR, want_bf16=True)
    ref = orc.gemm_dgrad(bits(dY), bits(W))
    assert np.array_equal(u32(dX.cpu().numpy()), u32(ref))
    assert np.array_equal(bits(dXb), orc.f32_to_bf16(ref))


@pytest.mark.parametrize("M,N,K", [(512, 4096, 2048), (77, 1024, 300)])
def test_gemm_dgrad_mfma(orc, M, N, K):
    dY = inputs.normal_bf16((M, N), 10200 + M, device=DEV)
    W = inputs.normal_bf16((N, K), 10201 + M, std=0.02, device=DEV)
    say("dgrad mfma", M, N, K)
    dX, _ = tb.tbik_gemm_dgrad(dY, W)
    # the same tree GEMM as the forward call on the transposed weight
    ref, _ = tb.tbik_gemm(dY, W.t().contiguous(), ws=None)
    assert torch.equal(dX.view(torch.int32), ref.view(torch.int32))
    # row subsets (batch invariance of the input gradient)
    sub, _ = tb.tbik_gemm_dgrad(dY[5:9], W)
    assert torch.equal(sub.view(torch.int32), dX[5:9].view(torch.int32))
    exact = orc.gemm_f64(bits(dY), np.ascontiguousarray(bits(W).T))
    err = np.abs(dX.cpu().numpy().astype(np.float64) - exact).max() / np.abs(exact).max()
    assert err <= 1e-5, err


@pytest.mark.parametrize("M,N,K,dps", [(256, 64, 96, (1, 2, 4)), (512, 40, 130, (1, 8))])
def test_gemm_wgrad_scalar_bitexact(orc, M, N, K, dps):
    dY = inputs.normal_bf16((M, N), 10300 + M)
    X = inputs.normal_bf16((M, K), 10301 + M)
    say("wgrad scalar", M, N, K)
    for dp in dps:
        dW, parts = tb.tbik_gemm_wgrad(dY.to(DEV), X.to(DEV), dp=dp, leaf_mode=tb.LEAF_SCALAR)
        ref, refp = orc.gemm_wgrad(bits(dY), bits(X), dp=dp)
        assert np.array_equal(u32(dW.cpu().numpy()), u32(ref)), dp
        if dp > 1:
            assert np.array_equal(u32(parts.cpu().numpy()), u32(refp)), dp


@pytest.mark.parametrize("M,N,K", [(4096, 2048, 2048), (1024, 5632, 512)])
def test_gemm_wgrad_mfma_dp_invariant(orc, M, N, K):
    dY = inputs.normal_bf16((M, N), 10400 + N, device=DEV)
    X = inputs.normal_bf16((M, K), 10401 + N, device=DEV)
    say("wgrad mfma", M, N, K)
    ref, _ = tb.tbik_gemm_wgrad(dY, X, dp=1)
    for dp in (2, 4, 8):
        dW, _ = tb.tbik_gemm_wgrad(dY, X, dp=dp)
        assert torch.equal(dW.view(torch.int32), ref.view(torch.int32)), dp
    rows = np.arange(0, N, max(1, N // 16))
    cols = np.arange(0, K, max(1, K // 16))
    dYt = np.ascontiguousarray(bits(dY).T)
    Xt = np.ascontiguousarray(bits(X).T)
    exact = orc.gemm_f64(dYt[rows], Xt[cols])
    got = ref.cpu().numpy()[np.ix_(rows, cols)].astype(np.float64)
    assert np.abs(got - exact).max() / np.abs(exact).max() <= 1e-5


def test_gemm_wgrad_integer_exact():
    M, N, K = 1024, 256, 192
    dY = inputs.integer_bf16((M, N), 10500).to(DEV)
    X = inputs.integer_bf16((M, K), 10501).to(DEV)
    dW, _ = tb.tbik_gemm_wgrad(dY, X, dp=4)
    exact = dY.float().cpu().numpy().astype(np.float64).T @ X.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(dW.cpu().numpy().astype(np.float64), exact)


@pytest.mark.parametrize("T,heads,d", [(2048, 16, 128), (33, 3, 64), (17, 6, 32)])
def test_rope_backward_bitexact(orc, T, heads, d):
    dy = inputs.normal_bf16((T, heads, d), 10600 + T)
    pos = inputs.positions(T, 32768, seed=13)
    c, s = orc.rope_table(1e6, d, 32768)
    say("rope backward", T, heads, d)
    dx = tb.tbik_rope_backward(dy.to(DEV), pos.to(DEV), torch.from_numpy(c).to(DEV),
                               torch.from_numpy(s).to(DEV))
    assert np.array_equal(bits(dx), orc.rope_backward(bits(dy), pos.numpy(), c, s))


@pytest.mark.parametrize("rows,cols", [(256, 5632), (3, 17)])
def test_swiglu_backward_bitexact(orc, rows, cols):
    g = inputs.normal_bf16((rows, cols), 10700 + rows, std=3.0)
    u = inputs.normal_bf16((rows, cols), 10701 + rows)
    d = inputs.normal_bf16((rows, cols), 10702 + rows)
    say("swiglu backward", rows, cols)
    dg, du = tb.tbik_swiglu_backward(g.to(DEV), u.to(DEV), d.to(DEV))
    rg, ru = orc.swiglu_backward(bits(g), bits(u), bits(d))
    assert np.array_equal(bits(dg), rg)
    assert np.array_equal(bits(du), ru)


def test_swiglu_backward_all_bf16_gates(orc):
    g = inputs.from_bits(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256))
    u = inputs.normal_bf16(g.shape, 10800)
    d = inputs.normal_bf16(g.shape, 10801)
    say("swiglu backward all gates")
    dg, du = tb.tbik_swiglu_backward(g.to(DEV), u.to(DEV), d.to(DEV))
    rg, ru = orc.swiglu_backward(bits(g), bits(u), bits(d))
    for got, ref in ((bits(dg), rg), (bits(du), ru)):
        nan_g = (got & 0x7FFF) > 0x7F80
        nan_r = (ref & 0x7FFF) > 0x7F80
        assert np.array_equal(nan_g, nan_r)
        assert np.array_equal(got[~nan_r], ref[~nan_r])


@pytest.mark.parametrize("rows,H,with_dr", [(64, 4096, True), (512, 4096, False),
                                            (4096, 4096, True), (128, 5120, True),
                                            (192, 1000, True), (64, 64, False),
                                            (64, 65534, True), (64, 10001, False),
                                            (128, 65535, True)])
def test_rmsnorm_backward_bitexact(orc, rows, H, with_dr):
    x = inputs.outlier_bf16((rows, H), 10900 + H)
    r = inputs.outlier_bf16((rows, H), 10901 + H)
    w = inputs.normal_bf16((H,), 10902 + H, std=0.1, mean=1.0)
    dy = inputs.normal_bf16((rows, H), 10903 + H)
    dr = inputs.normal_bf16((rows, H), 10904 + H, std=0.5) if with_dr else None
    say("rmsnorm backward", rows, H, with_dr)
    T = orc.lib().or_tree_T(rows // 64)
    for dp in [q for q in (1, 2, 4, 8) if T % q == 0]:
        dh, dw, shards = tb.tbik_rmsnorm_backward(
            x.to(DEV), r.to(DEV), w.to(DEV), dy.to(DEV), None if dr is None else dr.to(DEV),
            1e-6, dp=dp)
        rh, rw, rs = orc.rmsnorm_backward(bits(x), bits(r), bits(w), bits(dy),
                                          None if dr is None else bits(dr), 1e-6, dp=dp)
        assert np.array_equal(bits(dh), rh), dp
        assert np.array_equal(u32(dw.cpu().numpy()), u32(rw)), dp
        assert np.array_equal(u32(shards.cpu().numpy()), u32(rs)), dp


def test_rmsnorm_backward_without_dw(orc):
    rows, H = 7, 4096                                  # not a multiple of 64: no dw
    x = inputs.outlier_bf16((rows, H), 11000)
    r = inputs.outlier_bf16((rows, H), 11001)
    w = inputs.normal_bf16((H,), 11002, std=0.1, mean=1.0)
    dy = inputs.normal_bf16((rows, H), 11003)
    dh, dw, _ = tb.tbik_rmsnorm_backward(x.to(DEV), r.to(DEV), w.to(DEV), dy.to(DEV),
                                         want_dw=False)
    rh, _, _ = orc.rmsnorm_backward(bits(x), bits(r), bits(w), bits(dy), None, 1e-6,
                                    want_dw=False)
    assert dw is None and np.array_equal(bits(dh), rh)
