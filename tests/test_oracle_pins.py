"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test ties one oracle function to something the pages or mathematics
fix: hand-derived worked examples (tests/golden), exhaustive checks of the
primitives, exact results on integer data, binary64 references within a
stated error bound, closed forms, and the invariance the method promises
(bit-identical results for every tensor-parallel split; TBIK summary page,
Abstract).  A negative control shows the checks can see order changes.
"""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

from tp_invariant_numerics_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
U32 = 2.0 ** -24          # unit roundoff of binary32


def gamma(n):
    return n * U32 / (1 - n * U32)


def bf16_ulp(v):
    """Spacing of the bf16 grid at |v| (v float64 array)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def f32_bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# --------------------------------------------------------------------------
# premise: binary floating-point addition is not associative
# (IsoExec brief section 壹; nondeterminism note section 2)
# --------------------------------------------------------------------------
def test_premise_nonassociative():
    assert (0.1 + 0.2) + 0.3 != 0.1 + (0.2 + 0.3)
    a, b, c = np.float32(2.0 ** 24), np.float32(1.0), np.float32(1.0)
    assert (a + b) + c != a + (b + c)


# --------------------------------------------------------------------------
# primitives: exhaustive over every fp32 input / bf16 pair
# --------------------------------------------------------------------------
_PINS = None


def _pins_binary():
    global _PINS
    if _PINS is None:
        out = os.path.join(ROOT, "_build")
        os.makedirs(out, exist_ok=True)
        exe = os.path.join(out, "pins")
        subprocess.run(["gcc", "-O2", "-pthread", "-ffp-contract=off",
                        os.path.join(ROOT, "tests", "c", "pins.c"), "-o", exe, "-ldl", "-lm"],
                       check=True)
        _PINS = exe
    return _PINS


def _run_pins(orc, mode):
    from oracle import build as ob
    nth = str(min(16, os.cpu_count() or 1))
    r = subprocess.run([_pins_binary(), ob.LIB, mode, nth], check=True, capture_output=True,
                       text=True)
    kv = dict(tok.split("=") for tok in r.stdout.split())
    return float(kv["max_ulp"]), int(kv["bad"]), kv["worst"]


@pytest.mark.parametrize("mode", ["exp", "log"])
def test_explog_exhaustive_within_one_ulp(orc, mode):
    # EXP/LOG are library-defined (Cody-Waite + Taylor); every finite fp32
    # input is checked against binary64 libm: error < 1 ulp of binary32.
    mx, bad, worst = _run_pins(orc, mode)
    assert bad == 0, worst
    assert mx < 1.0, (mx, worst)


def test_bf16_products_exact_in_fp32(orc):
    # all 2^32 pairs of bf16 patterns; 8-bit significands multiply into at
    # most 16 bits (rounding-alignment article: bf16 keeps 7 stored bits)
    mx, bad, worst = _run_pins(orc, "prod")
    assert bad == 0, worst


def test_bf16_rounding_exhaustive(orc):
    mx, bad, worst = _run_pins(orc, "rne")
    assert bad == 0, worst


def test_explog_special_values(orc):
    e = orc.expf([0.0, -0.0, np.inf, -np.inf, np.nan, 89.5, -104.5, 88.0, -87.0])
    assert e[0] == 1.0 and e[1] == 1.0
    assert np.isposinf(e[2]) and e[3] == 0.0 and np.isnan(e[4])
    assert np.isposinf(e[5]) and e[6] == 0.0
    assert np.isfinite(e[7]) and e[8] > 0
    lg = orc.logf([1.0, 0.0, -1.0, np.inf, np.nan, 2.0 ** -149, 2.0 ** 127])
    assert lg[0] == 0.0 and np.isneginf(lg[1]) and np.isnan(lg[2])
    assert np.isposinf(lg[3]) and np.isnan(lg[4])
    assert abs(lg[5] - (-149 * math.log(2))) <= 2 * np.spacing(np.float32(103.0))
    assert abs(lg[6] - (127 * math.log(2))) <= np.spacing(np.float32(88.0))
    # EXP(k ln2) for integer k lands within 1 ulp of 2^k
    ks = np.arange(-120, 120)
    y = orc.expf((ks * math.log(2)).astype(np.float32))
    ref = np.exp(np.float32(ks * math.log(2)).astype(np.float64))
    assert np.all(np.abs(y - ref) <= np.spacing(np.abs(ref).astype(np.float32)))


# --------------------------------------------------------------------------
# the tree
# --------------------------------------------------------------------------
def _read_golden(name):
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(t) for t in line.split()])
    return rows


def test_tree_T():
    import oracle
    assert [oracle.tree_T(n) for n in (1, 2, 3, 6, 7, 12, 28, 224, 64, 16, 151936, 32000)] == \
        [1, 2, 1, 2, 1, 4, 4, 8, 8, 8, 8, 8]


def test_tree_structure_probes_golden(orc):
    for n, big, expected in _read_golden("tree_probes.txt"):
        v = np.ones(n, np.float32)
        v[big] = 2.0 ** 24
        got = orc.tree(v)
        assert got == np.float32(expected), (n, big, float(got), expected)


def _stream_counter(v):
    """PAIR evaluated as a streaming binary counter with a right fold at the
    end -- the form a GPU kernel uses when leaves arrive one at a time."""
    stack = []          # (level, value), strictly decreasing levels
    for x in v:
        node, lvl = np.float32(x), 0
        while stack and stack[-1][0] == lvl:
            node = np.float32(stack.pop()[1] + node)
            lvl += 1
        stack.append((lvl, node))
    acc = stack.pop()[1]
    while stack:
        acc = np.float32(stack.pop()[1] + acc)
    return acc


def test_pair_equals_streaming_counter(orc):
    rng = np.random.default_rng(1)
    for n in list(range(1, 300)) + [511, 512, 513, 1187, 1000, 2048, 4000]:
        v = rng.standard_normal(n).astype(np.float32) * np.float32(1e3) ** rng.standard_normal(n).astype(np.float32)
        assert f32_bits(orc.pair(v)) == f32_bits(_stream_counter(v)), n


@pytest.mark.parametrize("n", [8, 16, 24, 64, 224, 4096, 18992 * 8, 4000 * 8, 56, 88])
def test_tree_tp_invariant(orc, n):
    rng = np.random.default_rng(n)
    v = (rng.standard_normal(n) * np.exp(rng.standard_normal(n) * 3)).astype(np.float32)
    ref = orc.tree(v)
    T = orc.tree_T(n)
    tp = 1
    while tp <= T:
        r, nodes = orc.tree_sharded(v, tp)
        assert f32_bits(r) == f32_bits(ref), (n, tp)
        # the shard nodes combine by a perfect tree (hand-expanded)
        if tp == 2:
            assert f32_bits(np.float32(nodes[0] + nodes[1])) == f32_bits(ref)
        if tp == 4:
            assert f32_bits(np.float32(np.float32(nodes[0] + nodes[1]) +
                                       np.float32(nodes[2] + nodes[3]))) == f32_bits(ref)
        tp *= 2


def test_tree_exact_on_integers(orc):
    rng = np.random.default_rng(7)
    for n in (1, 5, 28, 224, 1000, 4096, 18992):
        v = rng.integers(-1000, 1000, n)
        assert orc.tree(v.astype(np.float32)) == np.float32(int(v.sum())), n


def test_tree_error_within_depth_bound(orc):
    rng = np.random.default_rng(3)
    for n in (28, 224, 4096, 18992 * 8):
        v = (rng.standard_normal(n) * np.exp(rng.standard_normal(n))).astype(np.float32)
        exact = math.fsum(v.astype(np.float64))
        T = orc.tree_T(n)
        depth = math.ceil(math.log2(n // T)) + int(math.log2(T))
        bound = gamma(depth) * float(np.abs(v.astype(np.float64)).sum())
        assert abs(float(orc.tree(v)) - exact) <= bound, n


def test_negative_control_order_matters(orc):
    # a sequential sum differs from the tree on ordinary data: the bitwise
    # checks of this suite can see a change of summation order
    rng = np.random.default_rng(11)
    v = rng.standard_normal(4096).astype(np.float32)
    seq = np.float32(0)
    for x in v:
        seq = np.float32(seq + x)
    assert f32_bits(seq) != f32_bits(orc.tree(v))


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------
def _bits(t):
    return inputs.bits(t)


def test_gemm_leaf_order_probes_golden(orc):
    for K, big, expected in _read_golden("gemm_leaf_probes.txt"):
        A = np.full((1, K), 0x3F80, np.uint16)          # bf16 1.0
        W = np.full((1, K), 0x3F80, np.uint16)
        W[0, big] = 0x4B80                               # bf16 2^24
        C = orc.gemm(A, W, nthreads=1)
        assert C[0, 0] == np.float32(expected), (K, big, float(C[0, 0]))


@pytest.mark.parametrize("M,N,K", [(3, 5, 64), (8, 8, 512), (4, 7, 448), (2, 3, 1792)])
def test_gemm_matches_binary64_within_bound(orc, M, N, K):
    A = _bits(inputs.normal_bf16((M, K), 10 + K))
    W = _bits(inputs.normal_bf16((N, K), 20 + K))
    C = orc.gemm(A, W)
    a = orc.bf16_to_f32(A).astype(np.float64)
    w = orc.bf16_to_f32(W).astype(np.float64)
    exact = np.array([[math.fsum(a[i] * w[j]) for j in range(N)] for i in range(M)])
    nb = K // 64
    T = orc.tree_T(nb)
    d = math.ceil(math.log2(max(1, nb // T))) + int(math.log2(T))
    bound = gamma(64 + d) * (np.abs(a) @ np.abs(w).T)
    assert np.all(np.abs(C - exact) <= bound)
    # a transposed operand or a dropped term would break this by far
    assert np.max(np.abs(C - exact)) < 1e-4 * np.max(np.abs(exact))


def test_gemm_exact_on_integers(orc):
    A = _bits(inputs.integer_bf16((6, 1024), 1))
    W = _bits(inputs.integer_bf16((9, 1024), 2))
    C = orc.gemm(A, W)
    ai = orc.bf16_to_f32(A).astype(np.int64)
    wi = orc.bf16_to_f32(W).astype(np.int64)
    assert np.array_equal(C.astype(np.int64), ai @ wi.T)


@pytest.mark.parametrize("K,tps", [(1024, (1, 2, 4, 8)), (14336, (1, 2, 4, 8)),
                                   (64 * 28, (1, 2, 4)), (64 * 12, (1, 2, 4))])
def test_gemm_tpsim_bit_identical(orc, K, tps):
    A = _bits(inputs.normal_bf16((5, K), 30))
    W = _bits(inputs.normal_bf16((6, K), 31, std=0.02))
    ref = orc.gemm(A, W)
    for tp in tps:
        C, parts = orc.gemm_tpsim(A, W, tp)
        assert np.array_equal(f32_bits(C), f32_bits(ref)), tp
        assert parts.shape == (tp, 5, 6)


def test_gemm_tp_rejects_misaligned_split(orc):
    A = np.zeros((1, 64 * 28), np.uint16)
    W = np.zeros((1, 64 * 28), np.uint16)
    with pytest.raises(ValueError):
        orc.gemm_tpsim(A, W, 8)          # 28 leaves: T = 4


def test_gemm_shard_partial_is_slice_gemm_when_groups_are_powers_of_two(orc):
    # K=1024: 16 leaves, T=8, G=2 -> the tree is a perfect binary tree, and
    # a shard of K/tp columns is itself a perfect tree: the shard partial is
    # the GEMM of that K slice (row-parallel partial sums, distributed-
    # training note 2.1.1)
    A = _bits(inputs.normal_bf16((4, 1024), 40))
    W = _bits(inputs.normal_bf16((3, 1024), 41))
    for tp in (2, 4, 8):
        _, parts = orc.gemm_tpsim(A, W, tp)
        ks = 1024 // tp
        for t in range(tp):
            sl = orc.gemm(np.ascontiguousarray(A[:, t * ks:(t + 1) * ks]),
                          np.ascontiguousarray(W[:, t * ks:(t + 1) * ks]))
            assert np.array_equal(f32_bits(parts[t]), f32_bits(sl)), (tp, t)


def test_gemm_rows_independent(orc):
    A = _bits(inputs.normal_bf16((16, 1024), 50))
    W = _bits(inputs.normal_bf16((8, 1024), 51))
    full = orc.gemm(A, W)
    for rows in ([0], [3, 7], list(range(5, 16))):
        sub = orc.gemm(np.ascontiguousarray(A[rows]), W)
        assert np.array_equal(f32_bits(sub), f32_bits(full[rows]))


def test_gemm_sampled_equals_full(orc):
    A = _bits(inputs.normal_bf16((7, 640), 60))
    W = _bits(inputs.normal_bf16((9, 640), 61))
    full = orc.gemm(A, W)
    rows = np.array([0, 6, 3, 2], np.int32)
    cols = np.array([8, 0, 4, 4], np.int32)
    assert np.array_equal(f32_bits(orc.gemm_sampled(A, W, rows, cols)), f32_bits(full[rows, cols]))


def test_negative_control_naive_tp_is_not_invariant(orc):
    A = _bits(inputs.normal_bf16((16, 14336), 70))
    W = _bits(inputs.normal_bf16((32, 14336), 71, std=0.02))
    n1 = orc.gemm_naive_tp(A, W, 1)
    n8 = orc.gemm_naive_tp(A, W, 8)
    assert np.count_nonzero(f32_bits(n1) != f32_bits(n8)) > 0
    t1 = orc.gemm(A, W)
    t8, _ = orc.gemm_tpsim(A, W, 8)
    assert np.array_equal(f32_bits(t1), f32_bits(t8))


# --------------------------------------------------------------------------
# residual RMSNorm (rounding-alignment article, "three nodes")
# --------------------------------------------------------------------------
def test_rmsnorm_constant_rows_closed_form(orc):
    H = 4096
    x = np.full((2, H), 0x3FC0, np.uint16)   # 1.5
    r = np.zeros((2, H), np.uint16)
    w = _bits(inputs.normal_bf16((H,), 80, std=0.1, mean=1.0))
    y, r_out = orc.rmsnorm_residual(x, r, w, 0.0)
    # ss = H * 2.25 exactly, mean = 2.25, rstd = fp32(1/1.5), h*rstd = 1.0 exactly?
    # (1.5 * fp32(2/3)) rounds to 1.0 in fp32, so y = bf16(w) = w exactly
    assert np.array_equal(r_out, x)
    assert np.array_equal(y[0], w) and np.array_equal(y[1], w)


def test_rmsnorm_matches_binary64(orc):
    rows, H = 64, 4096
    x = _bits(inputs.outlier_bf16((rows, H), 81))
    r = _bits(inputs.outlier_bf16((rows, H), 82))
    w = _bits(inputs.normal_bf16((H,), 83, std=0.1, mean=1.0))
    eps = 1e-6
    y, r_out = orc.rmsnorm_residual(x, r, w, eps)
    xf = orc.bf16_to_f32(x).astype(np.float64)
    rf = orc.bf16_to_f32(r).astype(np.float64)
    wf = orc.bf16_to_f32(w).astype(np.float64)
    h = xf + rf
    ref = h / np.sqrt((h * h).mean(axis=1, keepdims=True) + np.float64(np.float32(eps))) * wf
    yf = orc.bf16_to_f32(y).astype(np.float64)
    assert np.all(np.abs(yf - ref) <= bf16_ulp(ref) * 0.5 + 1e-5 * np.abs(ref) + 1e-30)
    assert np.all(np.abs(orc.bf16_to_f32(r_out) - h) <= bf16_ulp(h) * 0.5)


def test_rmsnorm_rows_independent(orc):
    x = _bits(inputs.normal_bf16((9, 512), 84))
    r = _bits(inputs.normal_bf16((9, 512), 85))
    w = _bits(inputs.normal_bf16((512,), 86, mean=1.0, std=0.1))
    y, _ = orc.rmsnorm_residual(x, r, w, 1e-6)
    y2, _ = orc.rmsnorm_residual(np.ascontiguousarray(x[4:6]), np.ascontiguousarray(r[4:6]), w, 1e-6)
    assert np.array_equal(y[4:6], y2)


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------
def test_rope_table_properties(orc):
    c, s = orc.rope_table(1e6, 128, 4096)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    # cos^2 + sin^2 = 1 up to two fp32 roundings
    assert np.max(np.abs(c.astype(np.float64) ** 2 + s.astype(np.float64) ** 2 - 1)) < 4 * U32
    # angle addition for p = 1000 + 2000 (binary64 identity, fp32 rounding)
    ca = c[1000].astype(np.float64); sa = s[1000].astype(np.float64)
    cb = c[2000].astype(np.float64); sb = s[2000].astype(np.float64)
    assert np.max(np.abs(c[3000] - (ca * cb - sa * sb))) < 1e-6
    # i = 0 frequency is 1 rad per position
    assert np.max(np.abs(c[:, 0] - np.cos(np.arange(4096.0)))) < 1e-7


def test_rope_position_zero_is_identity(orc):
    x = _bits(inputs.normal_bf16((4, 3, 128), 90))
    c, s = orc.rope_table(1e6, 128, 8)
    y = orc.rope(x, np.zeros(4, np.int32), c, s)
    assert np.array_equal(x, y)


def test_rope_matches_binary64_rotation(orc):
    T, heads, hd = 64, 4, 128
    x = _bits(inputs.normal_bf16((T, heads, hd), 91))
    pos = inputs.positions(T, 32768, seed=5).numpy() * 500 % 32768
    pos = pos.astype(np.int32)
    c, s = orc.rope_table(1e6, hd, 32768)
    y = orc.bf16_to_f32(orc.rope(x, pos, c, s)).astype(np.float64)
    xf = orc.bf16_to_f32(x).astype(np.float64)
    i = np.arange(hd // 2)
    ang = pos[:, None].astype(np.float64) * (1e6 ** (-(2.0 * i) / hd))[None, :]
    cc = np.cos(ang)[:, None, :]; ss = np.sin(ang)[:, None, :]
    a, b = xf[..., :hd // 2], xf[..., hd // 2:]
    ref = np.concatenate([a * cc - b * ss, b * cc + a * ss], axis=-1)
    tol = bf16_ulp(ref) * 0.5 + 4 * U32 * (np.abs(np.concatenate([a, b], -1)) + np.abs(np.concatenate([b, a], -1)))
    assert np.all(np.abs(y - ref) <= tol)


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------
def test_swiglu_closed_forms(orc):
    g = np.array([[0x0000, 0x8000, 0x3F80, 0xC2C8, 0x42C8, 0xC3C8]], np.uint16)  # 0,-0,1,-100,100,-400
    u = np.full_like(g, 0x4000)                                                  # 2.0
    y = orc.bf16_to_f32(orc.swiglu(g, u))
    assert y[0, 0] == 0.0 and y[0, 1] == 0.0
    assert y[0, 4] == 200.0                       # 100/(1+EXP(-100)) = 100
    assert y[0, 5] == 0.0                         # EXP(400) = inf -> -0
    assert abs(y[0, 2] - 2 / (1 + math.exp(-1))) <= 2.0 ** -7
    assert abs(y[0, 3]) < 1e-40


def test_swiglu_matches_binary64(orc):
    g = _bits(inputs.normal_bf16((32, 512), 92, std=3.0))
    u = _bits(inputs.normal_bf16((32, 512), 93))
    y = orc.bf16_to_f32(orc.swiglu(g, u)).astype(np.float64)
    gf = orc.bf16_to_f32(g).astype(np.float64)
    uf = orc.bf16_to_f32(u).astype(np.float64)
    ref = gf / (1 + np.exp(-gf)) * uf
    assert np.all(np.abs(y - ref) <= bf16_ulp(ref) * 0.5 + 8 * U32 * np.abs(ref) + 1e-38)


# --------------------------------------------------------------------------
# log-softmax + gather
# --------------------------------------------------------------------------
def test_logsoftmax_uniform_logits(orc):
    for V in (8, 1000, 32000, 151936):
        logits = np.full((2, V), 3.25, np.float32)
        lp, nodes = orc.logsoftmax_gather(logits, np.array([0, V - 1], np.int32))
        assert lp[0] == lp[1] == -orc.logf([np.float32(V)])[0]
        assert abs(lp[0] + math.log(V)) <= np.spacing(np.float32(math.log(V)))


def test_logsoftmax_dominant_logit(orc):
    V = 4096
    logits = np.zeros((1, V), np.float32)
    logits[0, 17] = 200.0
    lp, _ = orc.logsoftmax_gather(logits, np.array([17], np.int32))
    assert lp[0] == 0.0
    lp2, _ = orc.logsoftmax_gather(logits, np.array([18], np.int32))
    assert lp2[0] == -200.0


def test_logsoftmax_matches_binary64_and_tp_invariant(orc):
    M, V = 6, 32000
    rng = np.random.default_rng(12)
    logits = (rng.standard_normal((M, V)) * 4).astype(np.float32)
    tgt = rng.integers(0, V, M).astype(np.int32)
    lp1, n1 = orc.logsoftmax_gather(logits, tgt, tp=1)
    x = logits.astype(np.float64)
    m = x.max(axis=1, keepdims=True)
    ref = x[np.arange(M), tgt] - m[:, 0] - np.log(np.exp(x - m).sum(axis=1))
    assert np.all(np.abs(lp1 - ref) <= 1e-5 * np.maximum(1, np.abs(ref)))
    for tp in (2, 4, 8):
        lp, nodes = orc.logsoftmax_gather(logits, tgt, tp=tp)
        assert np.array_equal(f32_bits(lp), f32_bits(lp1)), tp
        # shard nodes are the sums over the shards' vocab slices
        sl = V // tp
        e = np.exp(x - m)
        for t in range(tp):
            assert np.allclose(nodes[:, t], e[:, t * sl:(t + 1) * sl].sum(axis=1), rtol=1e-5)


def test_logsoftmax_probabilities_sum_to_one(orc):
    V = 1000
    rng = np.random.default_rng(13)
    logits = (rng.standard_normal((1, V)) * 2).astype(np.float32)
    lps = np.array([orc.logsoftmax_gather(logits, np.array([t], np.int32))[0][0] for t in range(V)])
    assert abs(math.fsum(np.exp(lps.astype(np.float64))) - 1) < V * U32


# --------------------------------------------------------------------------
# causal softmax (decoder composition)
# --------------------------------------------------------------------------
def test_softmax_causal_properties(orc):
    L = 64
    rng = np.random.default_rng(14)
    S = (rng.standard_normal((L, L)) * 10).astype(np.float32)
    P = orc.bf16_to_f32(orc.softmax_causal(S, 0, np.float32(1 / math.sqrt(128))))
    assert P[0, 0] == 1.0 and np.all(P[0, 1:] == 0)
    assert np.all(np.triu(P, 1) == 0)
    rows = P.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(rows - 1) <= L * 2.0 ** -8)
    z = S.astype(np.float64) * np.float32(1 / math.sqrt(128))
    z = np.where(np.tril(np.ones((L, L))) > 0, z, -np.inf)
    ref = np.exp(z - z.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    assert np.all(np.abs(P - ref) <= bf16_ulp(ref) * 0.5 + 1e-6)
