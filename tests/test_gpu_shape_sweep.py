"""Seeded sweep over random GEMM shapes, row strides and tensor-parallel
sizes, bit for bit against the oracle with exact leaves.

Every row of A holds one nonzero entry per 64-wide K block, so each MFMA
leaf is a single exact product and the GEMM must reproduce the oracle's tree
exactly whatever launcher the shape selects (TBIK summary page, "technical
framework": local reduction, then the fixed binary tree).  The draws mix
boundary sizes (tile edges at 16, 32, 64, 128, 256 rows; one or two leaves;
the 11-, 22-, 28-leaf groups of real models) with uniform ones; the rows of A
and W carry padding whose contents differ from the data (a kernel that read
past K would change the result).  Sampled output columns keep the oracle's
share small.
"""
import numpy as np
import pytest
import torch

import tp_invariant_numerics_amd as tb
from tp_invariant_numerics_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"

EDGE_M = (1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513)
EDGE_N = (1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1024, 2047)
LEAVES = (1, 2, 3, 4, 5, 7, 8, 11, 16, 22, 28, 32, 44, 56, 64, 88, 112, 176, 224)


def _cases(n, seed):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        nb = int(g.choice(LEAVES))
        M = int(g.choice(EDGE_M)) if g.random() < 0.5 else int(g.integers(1, 600))
        N = int(g.choice(EDGE_N)) if g.random() < 0.5 else int(g.integers(1, 2600))
        T = 8 if nb % 8 == 0 else 4 if nb % 4 == 0 else 2 if nb % 2 == 0 else 1
        tp = int(g.choice([t for t in (1, 2, 4, 8) if T % t == 0]))
        pa, pw = int(g.choice([0, 8, 64])), int(g.choice([0, 8, 136]))
        out.append((i, M, N, 64 * nb, tp, pa, pw))
    return out


@pytest.mark.parametrize("i,M,N,K,tp,pa,pw", _cases(120, 20261203))
def test_random_shape_exact_leaves(orc, i, M, N, K, tp, pa, pw):
    print("case", i, "M", M, "N", N, "K", K, "tp", tp, "pad", pa, pw, flush=True)
    Af = inputs.one_per_block_bf16((M, K + pa), 15000 + i, spread=12)
    if pa:
        Af[:, K:] = inputs.normal_bf16((M, pa), 15500 + i) * 1000   # padding never read
    Wf = inputs.normal_bf16((N, K + pw), 16000 + i, device=DEV)
    if pw:
        Wf[:, K:] = float("nan")
    A = Af.to(DEV)[:, :K]
    W = Wf[:, :K]
    g = np.random.default_rng(i)
    cols = np.unique(np.concatenate([g.choice(N, min(N, 40), replace=False), [N - 1]]))
    ci = torch.from_numpy(cols).to(DEV)
    ref = orc.gemm(inputs.bits(Af[:, :K]), inputs.bits(W.index_select(0, ci)))
    refb = ref.view(np.uint32)
    C = tb.tbik_gemm(A, W)[0]
    got = C.index_select(1, ci).cpu().numpy().view(np.uint32)
    bad = np.argwhere(got != refb)
    assert bad.size == 0, ("tbik_gemm", "first mismatch", bad[0].tolist())
    if tp > 1:
        Ct = tb.tbik_gemm_tpsim(A, W, tp)[0]
        got = Ct.index_select(1, ci).cpu().numpy().view(np.uint32)
        bad = np.argwhere(got != refb)
        assert bad.size == 0, ("tbik_gemm_tpsim", tp, "first mismatch", bad[0].tolist())
