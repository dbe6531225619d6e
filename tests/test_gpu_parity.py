"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bit-exact for: the primitives (EXP, LOG, bf16 rounding), the scalar-leaf
GEMM and its simulated tensor-parallel partials, residual RMSNorm, RoPE,
SwiGLU, log-softmax + gather (including its shard sums) and the causal
softmax.  The MFMA-leaf GEMM has hardware-defined leaf bits, so it is held
to: bitwise invariance across tp and batch size (TBIK summary page,
Abstract), a normwise error <= 1e-5 against the binary64 product, an
elementwise summation bound, and exact results on integer data.
"""
import math

import numpy as np
import pytest
import torch

import tp_invariant_numerics_amd as tb
from tp_invariant_numerics_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    tb.lib()


def u32(x):
    return np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint32)


def f32_bits_t(t):
    return t.detach().cpu().numpy().view(np.uint32)


def same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


def bits(t):
    return inputs.bits(t)


# ------------------------------------------------------------------ primitives
@pytest.mark.parametrize("op", [tb.PRIM_EXP, tb.PRIM_LOG, tb.PRIM_BF16])
def test_primitives_bitexact(orc, op):
    rng = np.random.default_rng(100 + op)
    pats = rng.integers(0, 2 ** 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    if op == tb.PRIM_EXP:
        # dense coverage of the finite-result range too
        extra = np.linspace(-110, 95, 1 << 20, dtype=np.float32).view(np.uint32)
    elif op == tb.PRIM_LOG:
        extra = np.arange(1, 1 << 20, dtype=np.uint32)            # subnormals
    else:
        extra = np.arange(0, 1 << 20, dtype=np.uint32) * 4093
    x = np.concatenate([pats, extra]).view(np.float32)
    say("primitive", op, x.size)
    y = tb.tbik_primitive(op, torch.from_numpy(x).to(DEV)).cpu().numpy()
    if op == tb.PRIM_EXP:
        ref = orc.expf(x)
    elif op == tb.PRIM_LOG:
        ref = orc.logf(x)
    else:
        ref = orc.bf16_to_f32(orc.f32_to_bf16(x))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan)
    assert same_bits(y[~nan], ref[~nan])


def test_silu_all_bf16_gates(orc):
    """The gate activation on every one of the 2^16 bf16 gate values: the
    oracle's EXP, then IEEE fp32 add and division (numpy float32)."""
    g = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = orc.bf16_to_f32(g)
    say("silu all gates", x.size)
    y = tb.tbik_primitive(tb.PRIM_SILU, torch.from_numpy(x).to(DEV)).cpu().numpy()
    with np.errstate(all="ignore"):
        ref = x / (np.float32(1.0) + orc.expf(-x))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan)
    assert same_bits(y[~nan], ref[~nan])


def test_bf16_rounding_all_fp32():
    """fp32 -> bf16 round-to-nearest-even on all 2^32 fp32 patterns, in
    chunks: exact bits for every non-NaN input (numpy integer arithmetic on
    the bit pattern is the reference), a quiet NaN of the same sign for a NaN."""
    chunk = 1 << 28
    for c in range(1 << 32 >> 28):
        u = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint64).astype(np.uint32)
        say("bf16 all fp32, chunk", c)
        xd = torch.from_numpy(u.view(np.float32)).to(DEV)
        y = tb.tbik_primitive(tb.PRIM_BF16, xd).cpu().numpy().view(np.uint32)
        del xd
        nan = (u & 0x7FFFFFFF) > 0x7F800000
        ref = ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) & np.uint32(0xFFFF0000))
        assert np.array_equal(y[~nan], ref[~nan])
        yn = y[nan]
        assert np.all((yn & 0x7FC00000) == 0x7FC00000)       # quiet NaN
        assert np.array_equal(yn >> 31, u[nan] >> 31)          # sign kept
        assert np.all((yn & 0xFFFF) == 0)


# ------------------------------------------------------------------ GEMM
def _gen_gemm(M, N, K, seed, wstd=1.0):
    A = inputs.normal_bf16((M, K), seed)
    W = inputs.normal_bf16((N, K), seed + 1, std=wstd)
    return A, W


SCALAR_SHAPES = [(16, 256, 1024), (37, 83, 448), (1, 7, 64), (5, 33, 1792), (32, 64, 14336),
                 (3, 9, 64 * 11), (2, 5, 64 * 25)]


@pytest.mark.parametrize("M,N,K", SCALAR_SHAPES)
def test_gemm_scalar_bitexact(orc, M, N, K):
    A, W = _gen_gemm(M, N, K, 1000 + K)
    say("scalar gemm", M, N, K)
    C, Cb = tb.tbik_gemm(A.to(DEV), W.to(DEV), leaf_mode=tb.LEAF_SCALAR, want_bf16=True)
    ref = orc.gemm(bits(A), bits(W))
    assert same_bits(C.cpu().numpy(), ref)
    assert np.array_equal(bits(Cb), orc.f32_to_bf16(ref).reshape(M, N))


def test_gemm_scalar_leaf_probes_golden(orc):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "gemm_leaf_probes.txt")
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        K, big, expected = (int(t) for t in line.split())
        A = torch.ones((1, K), dtype=torch.bfloat16)
        W = torch.ones((1, K), dtype=torch.bfloat16)
        W[0, big] = 2.0 ** 24
        say("leaf probe", K, big)
        C, _ = tb.tbik_gemm(A.to(DEV), W.to(DEV), leaf_mode=tb.LEAF_SCALAR)
        assert C.item() == float(expected), (K, big, C.item())


@pytest.mark.parametrize("M,N,K,tps", [(16, 256, 1024, (1, 2, 4, 8)),
                                       (8, 40, 14336, (1, 2, 4, 8)),
                                       (5, 24, 64 * 28, (1, 2, 4)), (3, 5, 128, (1, 2)),
                                       (2, 1, 8 * 64 * 3, (1, 2, 4, 8))])
def test_gemm_tpsim_scalar_bitexact(orc, M, N, K, tps):
    A, W = _gen_gemm(M, N, K, 2000 + K, wstd=0.02)
    for tp in tps:
        say("tpsim scalar", M, N, K, tp)
        C, _, ws = tb.tbik_gemm_tpsim(A.to(DEV), W.to(DEV), tp, leaf_mode=tb.LEAF_SCALAR)
        refC, refws = orc.gemm_tpsim(bits(A), bits(W), tp)
        assert same_bits(C.cpu().numpy(), refC), tp
        assert same_bits(ws.cpu().numpy(), refws), tp


@pytest.mark.parametrize("M,N,K,tps", [(16, 256, 1024, (1, 2, 4, 8)),
                                       (1, 4096, 14336, (1, 2, 4, 8)),
                                       (32, 4096, 14336, (1, 2, 4, 8)),
                                       (256, 4096, 14336, (1, 2, 4, 8)),
                                       (77, 300, 64 * 28, (1, 2, 4)),
                                       (3, 5, 128, (1, 2)), (4, 17, 512, (1, 2, 4, 8)),
                                       (40, 1, 8 * 64 * 3, (1, 2, 4, 8))])
def test_gemm_mfma_tp_invariant(M, N, K, tps):
    A = inputs.normal_bf16((M, K), 3000 + M, device=DEV)
    W = inputs.normal_bf16((N, K), 3001 + M, std=0.02, device=DEV)
    say("mfma tp invariance", M, N, K)
    ref, _ = tb.tbik_gemm(A, W)
    refb = f32_bits_t(ref)
    for tp in tps:
        C, _, ws = tb.tbik_gemm_tpsim(A, W, tp)
        assert np.array_equal(f32_bits_t(C), refb), tp
        # the combine of the partials equals the top of the tree
        again = tb.tbik_tree_combine(ws)
        assert np.array_equal(f32_bits_t(again), refb), tp


@pytest.mark.parametrize("M,N,K", [(33, 4096, 14336), (256, 4096, 14336), (100, 2048, 2048),
                                   (77, 300, 5632), (130, 520, 4096), (32, 4096, 14336),
                                   (17, 1000, 14336), (16, 4096, 14336), (1, 4000, 14336)])
def test_gemm_split_k_workspace_same_bits(M, N, K):
    """tbik_gemm with its split-K workspace (nodes of the tree computed by
    separate workgroups, then the top of the tree) equals the one-launch
    result bit for bit, fp32 and bf16 outputs."""
    A = inputs.normal_bf16((M, K), 4300 + M, device=DEV)
    W = inputs.normal_bf16((N, K), 4301 + N, std=0.02, device=DEV)
    need = tb.tbik_gemm_workspace_bytes(M, N, K)
    say("split-K", M, N, K, "workspace bytes", need)
    assert need > 0
    C0, Cb0 = tb.tbik_gemm(A, W, want_bf16=True, ws=None)
    C1, Cb1 = tb.tbik_gemm(A, W, want_bf16=True)
    assert np.array_equal(f32_bits_t(C0), f32_bits_t(C1))
    assert torch.equal(Cb0.view(torch.int16), Cb1.view(torch.int16))
    _, Cb2 = tb.tbik_gemm(A, W, want_fp32=False, want_bf16=True)
    assert torch.equal(Cb0.view(torch.int16), Cb2.view(torch.int16))


def test_gemm_mfma_batch_invariant():
    K, N = 14336, 4096
    A = inputs.normal_bf16((256, K), 4000, device=DEV)
    W = inputs.normal_bf16((N, K), 4001, std=0.02, device=DEV)
    ref, _ = tb.tbik_gemm(A, W)
    refb = f32_bits_t(ref)
    bad = []
    for M in range(1, 257):
        C, _ = tb.tbik_gemm(A[:M], W)
        if not np.array_equal(f32_bits_t(C), refb[:M]):
            bad.append(M)
    assert not bad, bad
    # rows at other offsets and in permuted order
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(256, generator=g).to(DEV)
    C, _ = tb.tbik_gemm(A[perm].contiguous(), W)
    assert np.array_equal(f32_bits_t(C), refb[perm.cpu().numpy()])
    for off, M in ((3, 17), (100, 33), (200, 56), (255, 1)):
        C, _ = tb.tbik_gemm(A[off:off + M], W)
        assert np.array_equal(f32_bits_t(C), refb[off:off + M]), (off, M)


def test_gemm_mfma_column_slices_invariant():
    # column-parallel slices of W give the same bits as the full product
    K, N, M = 4096, 1024, 64
    A = inputs.normal_bf16((M, K), 4100, device=DEV)
    W = inputs.normal_bf16((N, K), 4101, std=0.02, device=DEV)
    ref = f32_bits_t(tb.tbik_gemm(A, W)[0])
    for lo, hi in ((0, 256), (256, 512), (8, 136), (1000, 1024)):
        C, _ = tb.tbik_gemm(A, W[lo:hi])
        assert np.array_equal(f32_bits_t(C), ref[:, lo:hi]), (lo, hi)


@pytest.mark.parametrize("M,N,K", [(16, 256, 1024), (64, 256, 14336), (40, 96, 4096),
                                   (1, 64, 14336), (300, 70, 2048), (5, 1, 64), (1, 1, 64),
                                   (2, 9, 192), (130, 3, 128)])
def test_gemm_mfma_accuracy(orc, M, N, K):
    A, W = _gen_gemm(M, N, K, 5000 + M, wstd=0.02)
    say("mfma accuracy", M, N, K)
    C = tb.tbik_gemm(A.to(DEV), W.to(DEV))[0].cpu().numpy().astype(np.float64)
    C64 = orc.gemm_f64(bits(A), bits(W))
    rel = np.max(np.abs(C - C64)) / np.max(np.abs(C64))
    assert rel <= 1e-5, rel
    # summation bound valid for any fp32 order, with u = 2^-23 to allow
    # truncating accumulation inside the matrix unit
    a = orc.bf16_to_f32(bits(A)).astype(np.float64)
    w = orc.bf16_to_f32(bits(W)).astype(np.float64)
    nb = K // 64
    T = orc.tree_T(nb)
    d = math.ceil(math.log2(max(1, nb // T))) + int(math.log2(T))
    n = 64 + d
    u = 2.0 ** -23
    bound = n * u / (1 - n * u) * (np.abs(a) @ np.abs(w).T)
    assert np.all(np.abs(C - C64) <= bound)


def test_gemm_mfma_integer_exact(orc):
    for (M, N, K) in ((16, 256, 1024), (33, 40, 14336)):
        A = inputs.integer_bf16((M, K), 6000 + M, -4, 4)
        W = inputs.integer_bf16((N, K), 6001 + M, -4, 4)
        C = tb.tbik_gemm(A.to(DEV), W.to(DEV))[0].cpu().numpy()
        ai = A.float().numpy().astype(np.int64)
        wi = W.float().numpy().astype(np.int64)
        assert np.array_equal(C.astype(np.int64), ai @ wi.T)


def test_gemm_mfma_bf16_output_is_rounded_fp32(orc):
    A, W = _gen_gemm(48, 200, 2048, 7000)
    C, Cb = tb.tbik_gemm(A.to(DEV), W.to(DEV), want_bf16=True)
    assert np.array_equal(bits(Cb), orc.f32_to_bf16(C.cpu().numpy()).reshape(48, 200))
    _, Cb2 = tb.tbik_gemm(A.to(DEV), W.to(DEV), want_fp32=False, want_bf16=True)
    assert np.array_equal(bits(Cb2), bits(Cb))


def test_gemm_strided_batched_equals_single(orc):
    B, M, N, K = 3, 40, 72, 512
    A = inputs.normal_bf16((B, M, K), 7100, device=DEV)
    W = inputs.normal_bf16((B, N, K), 7101, device=DEV)
    C, _ = tb.tbik_gemm_strided_batched(A, W)
    Cs, _ = tb.tbik_gemm_strided_batched(A, W, leaf_mode=tb.LEAF_SCALAR)
    for b in range(B):
        one, _ = tb.tbik_gemm(A[b], W[b])
        assert np.array_equal(f32_bits_t(C[b]), f32_bits_t(one))
        assert same_bits(Cs[b].cpu().numpy(), orc.gemm(bits(A[b]), bits(W[b])))


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("rows,H", [(1, 4096), (7, 4096), (256, 4096), (4096, 4096),
                                    (5, 2048), (3, 5120), (4, 1000), (9, 96), (2, 8), (3, 4104),
                                    (3, 64), (2, 512), (2, 16384), (2, 65536), (3, 1),
                                    (2, 24576), (2, 65534), (3, 65535), (2, 10001), (2, 8193),
                                    (2, 49154)])
def test_rmsnorm_bitexact(orc, rows, H):
    x = inputs.outlier_bf16((rows, H), 8000 + H)
    r = inputs.outlier_bf16((rows, H), 8001 + H)
    w = inputs.normal_bf16((H,), 8002 + H, std=0.1, mean=1.0)
    say("rmsnorm", rows, H)
    y, r_out = tb.tbik_rmsnorm_residual(x.to(DEV), r.to(DEV), w.to(DEV), 1e-6)
    ry, rr = orc.rmsnorm_residual(bits(x), bits(r), bits(w), 1e-6)
    assert np.array_equal(bits(y), ry)
    assert np.array_equal(bits(r_out), rr)


def test_rmsnorm_rows_invariant():
    x = inputs.outlier_bf16((512, 4096), 8100, device=DEV)
    r = inputs.outlier_bf16((512, 4096), 8101, device=DEV)
    w = inputs.normal_bf16((4096,), 8102, std=0.1, mean=1.0, device=DEV)
    y, _ = tb.tbik_rmsnorm_residual(x, r, w)
    for lo, hi in ((0, 1), (5, 6), (100, 357)):
        y2, _ = tb.tbik_rmsnorm_residual(x[lo:hi], r[lo:hi], w)
        assert torch.equal(y2.view(torch.int16), y[lo:hi].view(torch.int16))


# ------------------------------------------------------------------ RoPE
@pytest.mark.parametrize("T,heads,d", [(2048, 16, 128), (33, 3, 64), (5, 1, 8), (17, 6, 32),
                                        (9, 2, 8), (3, 2, 1024), (4, 3, 1016), (2, 64, 128)])
def test_rope_bitexact(orc, T, heads, d):
    x = inputs.normal_bf16((T, heads, d), 9000 + T)
    pos = inputs.positions(T, 32768, seed=9)
    pos = torch.from_numpy((pos.numpy().astype(np.int64) * 13 % 32768).astype(np.int32))
    c, s = orc.rope_table(1e6, d, 32768)
    say("rope", T, heads, d)
    y = tb.tbik_rope(x.to(DEV), pos.to(DEV), torch.from_numpy(c).to(DEV),
                     torch.from_numpy(s).to(DEV))
    ref = orc.rope(bits(x), pos.numpy(), c, s)
    assert np.array_equal(bits(y), ref)


def test_rope_in_place(orc):
    x = inputs.normal_bf16((64, 4, 128), 9100)
    pos = inputs.positions(64, 32768, seed=3)
    c, s = orc.rope_table(1e6, 128, 32768)
    xd = x.to(DEV)
    tb.tbik_rope(xd, pos.to(DEV), torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV), y=xd)
    assert np.array_equal(bits(xd), orc.rope(bits(x), pos.numpy(), c, s))


# ------------------------------------------------------------------ SwiGLU
@pytest.mark.parametrize("rows,cols", [(64, 14336), (4096, 14336), (3, 17), (5, 40)])
def test_swiglu_bitexact(orc, rows, cols):
    g = inputs.normal_bf16((rows, cols), 9500 + rows, std=3.0)
    u = inputs.normal_bf16((rows, cols), 9501 + rows)
    say("swiglu", rows, cols)
    y = tb.tbik_swiglu(g.to(DEV), u.to(DEV))
    assert np.array_equal(bits(y), orc.swiglu(bits(g), bits(u)))


def test_swiglu_all_bf16_gates(orc):
    g = inputs.from_bits(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256))
    u = inputs.normal_bf16(g.shape, 9700)
    say("swiglu all gates")
    y = bits(tb.tbik_swiglu(g.to(DEV), u.to(DEV)))
    ref = orc.swiglu(bits(g), bits(u))
    nan_y = (y & 0x7FFF) > 0x7F80
    nan_r = (ref & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_y, nan_r)
    assert np.array_equal(y[~nan_r], ref[~nan_r])


def test_swiglu_extreme_gates(orc):
    vals = np.array([0, -0.0, 1, -1, 88, -88, 89, -89, 100, -100, 1e-30, -1e-30, 3e38, -3e38],
                    np.float32)
    g = torch.from_numpy(np.tile(vals, 8).reshape(8, -1)).to(torch.bfloat16)
    u = inputs.normal_bf16(g.shape, 9600)
    y = tb.tbik_swiglu(g.to(DEV), u.to(DEV))
    assert np.array_equal(bits(y), orc.swiglu(bits(g), bits(u)))


# ------------------------------------------------------------------ logprob path
def _block_max_ref(C):
    M, N = C.shape
    nb = (N + 63) // 64
    pad = torch.full((M, nb * 64), -float("inf"), dtype=torch.float32, device=C.device)
    pad[:, :N] = C
    return pad.view(M, nb, 64).amax(dim=2)


@pytest.mark.parametrize("M,N,K", [(512, 151936, 4096), (100, 1000, 2048), (8, 300, 1024),
                                   (33, 65, 64 * 28), (1024, 33000, 2048)])
def test_gemm_logits_row_maxima(M, N, K):
    """The LM-head GEMM with fused 64-column row maxima: C is bitwise the
    plain GEMM's, pmax is exactly the maximum of each block of C."""
    A = inputs.normal_bf16((M, K), 4400 + M, device=DEV)
    W = inputs.normal_bf16((N, K), 4401 + N, std=0.02, device=DEV)
    say("gemm_logits", M, N, K)
    C, pmax = tb.tbik_gemm_logits(A, W)
    ref, _ = tb.tbik_gemm(A, W)
    assert np.array_equal(f32_bits_t(C), f32_bits_t(ref))
    assert np.array_equal(f32_bits_t(pmax), f32_bits_t(_block_max_ref(ref)))


@pytest.mark.parametrize("tp", [1, 4])
def test_logprob_path_fused_max_bitexact(orc, tp):
    """LM-head GEMM with fused maxima + one-read log-softmax = the oracle's
    log-softmax of the same logits, bit for bit (shard sums too)."""
    M, K, V = 512, 4096, 151936
    A = inputs.normal_bf16((M, K), 4500, device=DEV)
    W = inputs.normal_bf16((V, K), 4501, std=0.02, device=DEV)
    tgt = inputs.uniform_int(M, V, 4502, device=DEV)
    say("logprob path fused max, tp", tp)
    logits, pmax = tb.tbik_gemm_logits(A, W)
    lp, ws = tb.tbik_logsoftmax_gather_pmax(logits, tgt, pmax, tp)
    ref, nodes = orc.logsoftmax_gather(logits.cpu().numpy(), tgt.cpu().numpy(), tp)
    assert same_bits(lp.cpu().numpy(), ref)
    assert same_bits(tb.logsoftmax_shard_nodes(ws, M, tp).cpu().numpy(), nodes)
    lp2, _ = tb.tbik_logsoftmax_gather(logits, tgt, tp)
    assert same_bits(lp.cpu().numpy(), lp2.cpu().numpy())


# ------------------------------------------------------------------ log-softmax
@pytest.mark.parametrize("M,V,tps", [(8, 151936, (1, 2, 4, 8)), (16, 32000, (1, 2, 4, 8)),
                                     (5, 1000, (1, 2, 4, 8)), (3, 12, (1, 2, 4)),
                                     (4, 7, (1,)), (2, 655104, (1, 8)), (2, 40943, (1,)),
                                     (3, 1, (1,)), (3, 50257, (1,)), (2, 100277, (1,)),
                                     (2, 71702, (1, 2)), (2, 655100, (1, 4))])
def test_logsoftmax_bitexact(orc, M, V, tps):
    rng = np.random.default_rng(V)
    logits = (rng.standard_normal((M, V)) * 3).astype(np.float32)
    tgt = rng.integers(0, V, M).astype(np.int32)
    ld = (V + 7) // 8 * 8
    dev_logits = torch.zeros((M, ld), dtype=torch.float32, device=DEV)
    dev_logits[:, :V] = torch.from_numpy(logits).to(DEV)
    for tp in tps:
        say("logsoftmax", M, V, tp)
        lp, ws = tb.tbik_logsoftmax_gather(dev_logits[:, :V], torch.from_numpy(tgt).to(DEV), tp)
        ref, nodes = orc.logsoftmax_gather(logits, tgt, tp)
        assert same_bits(lp.cpu().numpy(), ref), tp
        got_nodes = tb.logsoftmax_shard_nodes(ws, M, tp).cpu().numpy()
        assert same_bits(got_nodes, nodes), tp


@pytest.mark.parametrize("V", [32000, 1000])
def test_logsoftmax_special_values(orc, V):
    """Masked vocabulary (-inf), a +inf logit, a NaN logit, targets on masked
    entries: the same NaN pattern as the oracle and the same bits elsewhere
    (V = 32000 takes the 16-element chunk path, V = 1000 single elements)."""
    M = 6
    rng = np.random.default_rng(V + 1)
    logits = (rng.standard_normal((M, V)) * 3).astype(np.float32)
    logits[0, ::3] = -np.inf                  # a third of the vocabulary masked
    logits[1, 5] = np.inf
    logits[2, V // 2] = np.nan
    logits[3, :] = -np.inf
    logits[3, 7] = 1.0
    logits[4, -1] = 80.0                      # far above the rest of its row
    tgt = rng.integers(0, V, M).astype(np.int32)
    tgt[0] = 3                                # a masked entry: log-probability -inf
    tgt[3] = 7
    dev = torch.from_numpy(logits).to(DEV)
    for tp in (1, 4):
        say("logsoftmax special values", V, tp)
        lp, ws = tb.tbik_logsoftmax_gather(dev, torch.from_numpy(tgt).to(DEV), tp)
        ref, nodes = orc.logsoftmax_gather(logits, tgt, tp)
        got = lp.cpu().numpy()
        assert np.array_equal(np.isnan(got), np.isnan(ref)), tp
        ok = ~np.isnan(ref)
        assert same_bits(got[ok], ref[ok]), tp
        gn = tb.logsoftmax_shard_nodes(ws, M, tp).cpu().numpy()
        okn = ~np.isnan(nodes)
        assert np.array_equal(np.isnan(gn), np.isnan(nodes)), tp
        assert same_bits(gn[okn], nodes[okn]), tp


# ------------------------------------------------------------------ causal softmax
@pytest.mark.parametrize("B,Lq,Lk,offset", [(2, 512, 512, 0), (3, 64, 128, 64), (1, 9, 24, 0),
                                            (2, 130, 256, 0), (2, 64, 64, 0), (1, 512, 1024, 512),
                                            (1, 5, 10001, 9990), (1, 3, 65535, 65530),
                                            (1, 4, 16386, 16380)])
def test_softmax_causal_bitexact(orc, B, Lq, Lk, offset):
    rng = np.random.default_rng(Lk + offset)
    S = (rng.standard_normal((B, Lq, Lk)) * 30).astype(np.float32)
    scale = np.float32(1 / math.sqrt(128))
    say("softmax_causal", B, Lq, Lk, offset)
    P = tb.tbik_softmax_causal(torch.from_numpy(S).to(DEV), offset, float(scale))
    for b in range(B):
        assert np.array_equal(bits(P[b]), orc.softmax_causal(S[b], offset, scale))


# ------------------------------------------------------------------ real-TP building blocks
@pytest.mark.parametrize("leaf", [tb.LEAF_MFMA, tb.LEAF_SCALAR])
def test_gemm_shard_and_partials_match_tpsim(orc, leaf):
    M, N, K = 24, 96, 14336
    A = inputs.normal_bf16((M, K), 7200, device=DEV)
    W = inputs.normal_bf16((N, K), 7201, std=0.02, device=DEV)
    ref = f32_bits_t(tb.tbik_gemm(A, W, leaf_mode=leaf)[0])
    for tp in (1, 2, 4, 8):
        _, _, ws = tb.tbik_gemm_tpsim(A, W, tp, leaf_mode=leaf)
        parts = tb.tbik_gemm_tp_partials(A, W, tp, leaf_mode=leaf)
        assert np.array_equal(f32_bits_t(parts), f32_bits_t(ws)), tp
        ks = K // tp
        shards = torch.stack([tb.tbik_gemm_shard(A[:, t * ks:(t + 1) * ks].contiguous(),
                                                 W[:, t * ks:(t + 1) * ks].contiguous(),
                                                 K, tp, leaf_mode=leaf) for t in range(tp)])
        assert np.array_equal(f32_bits_t(shards), f32_bits_t(ws)), tp
        assert np.array_equal(f32_bits_t(tb.tbik_tree_combine(shards)), ref), tp
    if leaf == tb.LEAF_SCALAR:
        _, refws = orc.gemm_tpsim(bits(A.cpu()), bits(W.cpu()), 8)
        assert same_bits(parts.cpu().numpy(), refws)


@pytest.mark.parametrize("M,N", [(256, 4096), (300, 4000)])
def test_tp8_partials_of_paired_shards(M, N):
    """At these sizes the tp = 8 partials kernel streams two consecutive
    shards per workgroup; each partial must still be exactly that shard's
    node, as one rank computes it from its own K slice."""
    K, tp = 14336, 8
    A = inputs.normal_bf16((M, K), 7300 + M, device=DEV)
    W = inputs.normal_bf16((N, K), 7301 + N, std=0.02, device=DEV)
    say("tp8 paired partials", M, N, K)
    ws = tb.tbik_gemm_tp_partials(A, W, tp)
    ks = K // tp
    for t in range(tp):
        node = tb.tbik_gemm_shard(A[:, t * ks:(t + 1) * ks].contiguous(),
                                  W[:, t * ks:(t + 1) * ks].contiguous(), K, tp)
        assert np.array_equal(f32_bits_t(ws[t]), f32_bits_t(node)), t
    ref = f32_bits_t(tb.tbik_gemm(A, W)[0])
    assert np.array_equal(f32_bits_t(tb.tbik_tree_combine(ws)), ref)


# ------------------------------------------------------------------ unaligned strides
def test_rowops_unaligned_strides(orc):
    rows, H = 6, 4096
    x = inputs.outlier_bf16((rows, H), 7300)
    r = inputs.outlier_bf16((rows, H), 7301)
    w = inputs.normal_bf16((H,), 7302, std=0.1, mean=1.0)
    ry, rr = orc.rmsnorm_residual(bits(x), bits(r), bits(w), 1e-6)
    for pad in (1, 3, 4):
        xd = torch.zeros((rows, H + pad), dtype=torch.bfloat16, device=DEV)
        rd = torch.zeros_like(xd)
        xd[:, :H] = x.to(DEV)
        rd[:, :H] = r.to(DEV)
        yd = torch.zeros_like(xd)
        rod = torch.zeros_like(xd)
        tb.tbik_rmsnorm_residual(xd[:, :H], rd[:, :H], w.to(DEV), 1e-6, y=yd[:, :H],
                                 r_out=rod[:, :H])
        assert np.array_equal(bits(yd[:, :H]), ry), pad
        assert np.array_equal(bits(rod[:, :H]), rr), pad
    g = inputs.normal_bf16((5, 64), 7303, std=3.0)
    u = inputs.normal_bf16((5, 64), 7304)
    gd = torch.zeros((5, 67), dtype=torch.bfloat16, device=DEV)
    gd[:, :64] = g.to(DEV)
    out = tb.tbik_swiglu(gd[:, :64], u.to(DEV))
    assert np.array_equal(bits(out), orc.swiglu(bits(g), bits(u)))
    rng = np.random.default_rng(7305)
    logits = (rng.standard_normal((4, 32000)) * 3).astype(np.float32)
    tgt = rng.integers(0, 32000, 4).astype(np.int32)
    ld = torch.zeros((4, 32003), dtype=torch.float32, device=DEV)
    ld[:, :32000] = torch.from_numpy(logits).to(DEV)
    lp, _ = tb.tbik_logsoftmax_gather(ld[:, :32000], torch.from_numpy(tgt).to(DEV), 4)
    assert same_bits(lp.cpu().numpy(), orc.logsoftmax_gather(logits, tgt, 4)[0])


@pytest.mark.parametrize("M,K,N", [(2048, 2048, 4096), (2048, 1024, 4096), (4096, 2048, 2100),
                                   (4096, 4096, 2048)])
def test_gemm_whole_part_perfect_tree(orc, M, K, N):
    """Power-of-two groups: the part's tree is one perfect tree evaluated as a
    single compile-time group.  Same bits across tp and batch, accurate,
    and exact on integer data."""
    A = inputs.normal_bf16((M, K), 4600 + K, device=DEV)
    W = inputs.normal_bf16((N, K), 4601 + K, std=0.02, device=DEV)
    say("perfect-tree gemm", M, K, N)
    ref = f32_bits_t(tb.tbik_gemm(A, W, ws=None)[0])
    for tp in (2, 4, 8):
        assert np.array_equal(f32_bits_t(tb.tbik_gemm_tpsim(A, W, tp)[0]), ref), tp
    for m in (1, 33, 257):
        assert np.array_equal(f32_bits_t(tb.tbik_gemm(A[:m], W)[0]), ref[:m]), m
    Ai = inputs.integer_bf16((M, K), 4602).to(DEV)
    Wi = inputs.integer_bf16((N, K), 4603).to(DEV)
    Ci = tb.tbik_gemm(Ai, Wi)[0].cpu().numpy().astype(np.float64)
    exact = Ai.float().cpu().numpy().astype(np.float64) @ Wi.float().cpu().numpy().astype(np.float64).T
    assert np.array_equal(Ci, exact)


@pytest.mark.parametrize("M,F,K", [(4096, 5632, 2048), (100, 48, 2048), (257, 1040, 5632),
                                   (33, 16, 1024), (300, 2000, 14336)])
@pytest.mark.parametrize("rounding", ["once", "each_op"])
def test_gemm_swiglu_fused_equals_composition(M, F, K, rounding):
    """The gate/up GEMM with SwiGLU in its epilogue returns what the tree
    GEMM's bf16 output followed by the SwiGLU node returns, bit for bit."""
    A = inputs.normal_bf16((M, K), 7500 + M, device=DEV)
    W = inputs.normal_bf16((2 * F, K), 7501 + F, std=0.05, device=DEV)
    say("gemm+swiglu fused", M, F, K, rounding)
    H = tb.tbik_gemm_swiglu(A, W, rounding=rounding)
    _, gu = tb.tbik_gemm(A, W, want_fp32=False, want_bf16=True)
    ref = tb.tbik_swiglu(gu[:, :F], gu[:, F:], rounding=rounding)
    assert torch.equal(H.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("M", [1, 32, 256])
def test_downproj_full_size_sampled_accuracy(orc, M):
    """The row-parallel down projection at its full size (K = 14336,
    N = 4096) in the launch configurations the benchmark times: tp = 8
    simulated shards (paired shards per workgroup at M = 256, thin tiles at
    M <= 32) and tp = 1 with the split-K workspace.  Both give the same bits;
    sampled outputs are within 1e-5 normwise of the binary64 product."""
    K, N = 14336, 4096
    A = inputs.normal_bf16((M, K), 7400 + M, device=DEV)
    W = inputs.normal_bf16((N, K), 7401, std=0.02, device=DEV)
    say("down projection full size", M)
    C8 = f32_bits_t(tb.tbik_gemm_tpsim(A, W, 8)[0])
    C1 = f32_bits_t(tb.tbik_gemm(A, W)[0])
    assert np.array_equal(C8, C1)
    rows = np.arange(0, M, max(1, M // 8))
    cols = np.arange(3, N, 61)
    exact = orc.gemm_f64(bits(A[rows]), bits(W[cols]))
    got = C1.view(np.float32)[np.ix_(rows, cols)].astype(np.float64)
    assert np.abs(got - exact).max() / np.abs(exact).max() <= 1e-5


@pytest.mark.parametrize("M,N", [(4096, 2048), (256, 2048), (40, 520)])
def test_gemm_group11_schedule(orc, M, N):
    """K = 5632 (88 leaves, groups of 11, the decoder's down projection):
    the compile-time group schedule starts groups at leaf offsets that are
    not multiples of the ring depth.  Same bits for every tp and batch
    subset, exact on integer data, accurate on random data."""
    K = 5632
    A = inputs.normal_bf16((M, K), 4700 + M, device=DEV)
    W = inputs.normal_bf16((N, K), 4701 + N, std=0.02, device=DEV)
    say("group-11 gemm", M, N, K)
    ref = f32_bits_t(tb.tbik_gemm(A, W, ws=None)[0])
    assert np.array_equal(f32_bits_t(tb.tbik_gemm(A, W)[0]), ref)
    for tp in (2, 4, 8):
        assert np.array_equal(f32_bits_t(tb.tbik_gemm_tpsim(A, W, tp)[0]), ref), tp
    for m in (1, 31, 129):
        if m < M:
            assert np.array_equal(f32_bits_t(tb.tbik_gemm(A[:m], W)[0]), ref[:m]), m
    rows = np.arange(0, M, max(1, M // 16))
    cols = np.arange(0, N, max(1, N // 16))
    rr, cc = np.meshgrid(rows, cols, indexing="ij")
    exact = orc.gemm_f64(bits(A[rows]), bits(W[cols]))
    got = ref.view(np.float32)[rr, cc].astype(np.float64)
    assert np.abs(got - exact).max() / np.abs(exact).max() <= 1e-5
    Ai = inputs.integer_bf16((M, K), 4702).to(DEV)
    Wi = inputs.integer_bf16((N, K), 4703).to(DEV)
    Ci = tb.tbik_gemm(Ai, Wi)[0].cpu().numpy().astype(np.float64)
    Af = Ai.float().cpu().numpy().astype(np.float64)
    Wf = Wi.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(Ci[rr, cc], (Af[rows] @ Wf[cols].T))


# ------------------------------------------------------------------ rounding locations
# (rounding-alignment article, "three nodes": the misaligned stack rounds
# intermediates to bf16; TBIK_ROUND_EACH_OP is that stack as eager bf16
# arithmetic, bit-exact against the oracle's variant)
@pytest.mark.parametrize("rows,H", [(7, 4096), (300, 4096), (3, 5120), (2, 16384), (4, 1000)])
def test_rmsnorm_each_op_bitexact(orc, rows, H):
    x = inputs.outlier_bf16((rows, H), 8300 + H)
    r = inputs.outlier_bf16((rows, H), 8301 + H)
    w = inputs.normal_bf16((H,), 8302 + H, std=0.1, mean=1.0)
    say("rmsnorm each_op", rows, H)
    y, r_out = tb.tbik_rmsnorm_residual(x.to(DEV), r.to(DEV), w.to(DEV), 1e-6, rounding="each_op")
    ry, rr = orc.rmsnorm_residual(bits(x), bits(r), bits(w), 1e-6, rounding="each_op")
    assert np.array_equal(bits(y), ry)
    assert np.array_equal(bits(r_out), rr)
    y0, _ = tb.tbik_rmsnorm_residual(x.to(DEV), r.to(DEV), w.to(DEV), 1e-6)
    assert np.count_nonzero(bits(y0) != ry) > 0


@pytest.mark.parametrize("T,heads,d", [(2048, 16, 128), (33, 3, 64)])
def test_rope_each_op_bitexact(orc, T, heads, d):
    x = inputs.normal_bf16((T, heads, d), 9200 + T)
    pos = inputs.positions(T, 32768, seed=11)
    c, s = orc.rope_table(1e6, d, 32768)
    say("rope each_op", T, heads, d)
    y = tb.tbik_rope(x.to(DEV), pos.to(DEV), torch.from_numpy(c).to(DEV),
                     torch.from_numpy(s).to(DEV), rounding="each_op")
    assert np.array_equal(bits(y), orc.rope(bits(x), pos.numpy(), c, s, rounding="each_op"))


@pytest.mark.parametrize("rows,cols", [(512, 14336), (3, 17)])
def test_swiglu_each_op_bitexact(orc, rows, cols):
    g = inputs.normal_bf16((rows, cols), 9800 + rows, std=3.0)
    u = inputs.normal_bf16((rows, cols), 9801 + rows)
    say("swiglu each_op", rows, cols)
    y = tb.tbik_swiglu(g.to(DEV), u.to(DEV), rounding="each_op")
    assert np.array_equal(bits(y), orc.swiglu(bits(g), bits(u), rounding="each_op"))


# ------------------------------------------------------------------ alignment never changes the shapes
@pytest.mark.parametrize("V,ld,off", [(151936, 151937, 0), (151936, 151940, 1), (655104, 655105, 3),
                                      (32000, 32001, 1)])
def test_logsoftmax_unaligned_rows_accepted_and_bitexact(orc, V, ld, off):
    """Rows whose starts are not 16-byte aligned take element-wise loads of
    the same chunks: accepted exactly like aligned rows (the LM-head
    vocabulary at an odd row stride; V = 655104, the largest vocabulary the
    LDS staging takes, at an odd offset), with the oracle's bits."""
    M = 3
    rng = np.random.default_rng(V + ld)
    logits = (rng.standard_normal((M, V)) * 3).astype(np.float32)
    tgt = rng.integers(0, V, M).astype(np.int32)
    buf = torch.zeros((M * ld + off + 8,), dtype=torch.float32, device=DEV)
    view = buf[off:off + M * ld].view(M, ld)[:, :V]
    view.copy_(torch.from_numpy(logits).to(DEV))
    say("logsoftmax unaligned", V, ld, off)
    for tp in (1, 4):
        lp, ws = tb.tbik_logsoftmax_gather(view, torch.from_numpy(tgt).to(DEV), tp)
        ref, nodes = orc.logsoftmax_gather(logits, tgt, tp)
        assert same_bits(lp.cpu().numpy(), ref), tp
        assert same_bits(tb.logsoftmax_shard_nodes(ws, M, tp).cpu().numpy(), nodes), tp


@pytest.mark.parametrize("H,off", [(4096, 1), (4104, 3), (4096, 2), (65536, 1), (5120, 5)])
def test_rmsnorm_unaligned_rows_accepted_and_bitexact(orc, H, off):
    rows = 3
    x = inputs.outlier_bf16((rows, H), 8500 + H)
    r = inputs.outlier_bf16((rows, H), 8501 + H)
    w = inputs.normal_bf16((H,), 8502 + H, std=0.1, mean=1.0)
    ld = H + 3
    say("rmsnorm unaligned", H, off)

    def place(t):
        buf = torch.zeros((rows * ld + off + 8,), dtype=torch.bfloat16, device=DEV)
        v = buf[off:off + rows * ld].view(rows, ld)[:, :H]
        if t is not None:
            v.copy_(t.to(DEV))
        return v

    xd, rd, yd, rod = place(x), place(r), place(None), place(None)
    wbuf = torch.zeros((H + off + 8,), dtype=torch.bfloat16, device=DEV)
    wd = wbuf[off:off + H]
    wd.copy_(w.to(DEV))
    tb.tbik_rmsnorm_residual(xd, rd, wd, 1e-6, y=yd, r_out=rod)
    ry, rr = orc.rmsnorm_residual(bits(x), bits(r), bits(w), 1e-6)
    assert np.array_equal(bits(yd), ry)
    assert np.array_equal(bits(rod), rr)
    # the backward pass at the same offsets: dh equal to the aligned call
    gy = inputs.normal_bf16((rows, H), 8503 + H)
    gyd = place(gy)
    dh_u, _, _ = tb.tbik_rmsnorm_backward(xd, rd, wd, gyd, want_dw=False)
    dh_a, _, _ = tb.tbik_rmsnorm_backward(x.to(DEV), r.to(DEV), w.to(DEV), gy.to(DEV), want_dw=False)
    assert torch.equal(dh_u.view(torch.int16), dh_a.view(torch.int16))


@pytest.mark.parametrize("Lq,Lk,lds_pad", [(40, 512, 1), (33, 96, 3), (64, 64, 1)])
def test_softmax_causal_unaligned_rows_bitexact(orc, Lq, Lk, lds_pad):
    rng = np.random.default_rng(Lk + lds_pad)
    S = (rng.standard_normal((1, Lq, Lk)) * 20).astype(np.float32)
    ld = Lk + lds_pad
    buf = torch.zeros((Lq * ld + 4,), dtype=torch.float32, device=DEV)
    Sv = buf[:Lq * ld].view(1, Lq, ld)[:, :, :Lk]
    Sv.copy_(torch.from_numpy(S).to(DEV))
    scale = np.float32(1 / math.sqrt(128))
    say("softmax_causal unaligned", Lq, Lk, lds_pad)
    P = tb.tbik_softmax_causal(Sv, 0, float(scale))
    assert np.array_equal(bits(P[0]), orc.softmax_causal(S[0], 0, scale))
