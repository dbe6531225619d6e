"""Seeded sweeps over random shapes of the row nodes, bit for bit against
the oracle: residual RMSNorm (TBIK summary page, Abstract: invariant
reduction primitives; alignment article, "three nodes"), RoPE and SwiGLU
(same article), and the log-softmax + gather with its shard sums, both with
its own row maxima and with 64-column maxima handed in (the LM-head path).
Sizes are drawn uniformly and from the edges where the kernels change form
(chunk widths, the register and LDS variants, one group, ragged groups)."""
import numpy as np
import pytest
import torch

import tp_invariant_numerics_amd as tb
from tp_invariant_numerics_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return inputs.bits(t)


def _same(a, b):
    """float32 arrays equal bit for bit, NaNs by NaN-ness."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


def _draw(g, edges, lo, hi):
    return int(g.choice(edges)) if g.random() < 0.5 else int(g.integers(lo, hi))


H_EDGES = (1, 2, 3, 7, 8, 16, 63, 64, 96, 127, 512, 1000, 2048, 2050, 4096, 4104, 5120, 8191, 8192)


@pytest.mark.parametrize("i", range(30))
def test_rmsnorm_random(orc, i):
    g = np.random.default_rng(31000 + i)
    rows, H = _draw(g, (1, 2, 5, 64, 255), 1, 300), _draw(g, H_EDGES, 1, 9000)
    x = inputs.outlier_bf16((rows, H), 31100 + i)
    r = inputs.outlier_bf16((rows, H), 31200 + i)
    w = inputs.normal_bf16((H,), 31300 + i, std=0.1, mean=1.0)
    print("rmsnorm", i, rows, H, flush=True)
    y, r_out = tb.tbik_rmsnorm_residual(x.to(DEV), r.to(DEV), w.to(DEV), 1e-6)
    ry, rr = orc.rmsnorm_residual(_bits(x), _bits(r), _bits(w), 1e-6)
    assert np.array_equal(_bits(y), ry)
    assert np.array_equal(_bits(r_out), rr)


@pytest.mark.parametrize("i", range(20))
def test_rope_random(orc, i):
    g = np.random.default_rng(32000 + i)
    d = int(g.choice([8, 16, 24, 32, 64, 96, 128, 256, 1016, 1024]))
    T, heads = _draw(g, (1, 2, 33), 1, 200), _draw(g, (1, 3, 16, 17), 1, 24)
    x = inputs.normal_bf16((T, heads, d), 32100 + i)
    pos = torch.from_numpy(g.integers(0, 32768, T).astype(np.int32))
    c, s = orc.rope_table(1e6, d, 32768)
    print("rope", i, T, heads, d, flush=True)
    y = tb.tbik_rope(x.to(DEV), pos.to(DEV), torch.from_numpy(c).to(DEV),
                     torch.from_numpy(s).to(DEV))
    assert np.array_equal(_bits(y), orc.rope(_bits(x), pos.numpy(), c, s))


@pytest.mark.parametrize("i", range(20))
def test_swiglu_random(orc, i):
    g = np.random.default_rng(33000 + i)
    rows, cols = _draw(g, (1, 2, 7), 1, 300), _draw(g, (1, 7, 8, 9, 15, 16, 17), 1, 20000)
    gate = inputs.normal_bf16((rows, cols), 33100 + i, std=3.0)
    up = inputs.normal_bf16((rows, cols), 33200 + i)
    print("swiglu", i, rows, cols, flush=True)
    y = tb.tbik_swiglu(gate.to(DEV), up.to(DEV))
    assert np.array_equal(_bits(y), orc.swiglu(_bits(gate), _bits(up)))


V_EDGES = (1, 2, 7, 8, 12, 16, 64, 1000, 1187, 32000, 40943, 40945, 50257, 100277, 128000,
           151936, 151937, 152070)


@pytest.mark.parametrize("i", range(30))
def test_logsoftmax_random(orc, i):
    g = np.random.default_rng(34000 + i)
    M, V = _draw(g, (1, 2, 3), 1, 24), _draw(g, V_EDGES, 1, 200000)
    T = next(t for t in (8, 4, 2, 1) if V % t == 0)
    tp = int(g.choice([t for t in (1, 2, 4, 8) if T % t == 0]))
    logits = (g.standard_normal((M, V)) * float(g.choice([0.5, 3.0, 20.0]))).astype(np.float32)
    tgt = g.integers(0, V, M).astype(np.int32)
    print("logsoftmax", i, M, V, tp, flush=True)
    lg = torch.from_numpy(logits).to(DEV)
    td = torch.from_numpy(tgt).to(DEV)
    ref, nodes = orc.logsoftmax_gather(logits, tgt, tp)
    lp, ws = tb.tbik_logsoftmax_gather(lg, td, tp)
    assert _same(lp.cpu().numpy(), ref)
    assert _same(tb.logsoftmax_shard_nodes(ws, M, tp).cpu().numpy(), nodes)
    # the same with 64-column row maxima handed in (what the LM-head GEMM writes)
    nb = (V + 63) // 64
    pad = torch.full((M, nb * 64), -float("inf"), device=DEV)
    pad[:, :V] = lg
    pmax = pad.view(M, nb, 64).amax(dim=2).contiguous()
    lp2, ws2 = tb.tbik_logsoftmax_gather_pmax(lg, td, pmax, tp)
    assert _same(lp2.cpu().numpy(), ref)
    assert _same(tb.logsoftmax_shard_nodes(ws2, M, tp).cpu().numpy(), nodes)
