"""Matrix-core GEMM bit for bit against the oracle, with exact leaves.

The MFMA leaf adds its 64 products in an order the hardware fixes, so on
general data only the leaves' bits are free.  Giving every row of A exactly
one nonzero entry per 64-wide K block makes every leaf a single exact
product: its bits no longer depend on that order, and everything above the
leaves -- the compile-time tree schedules of the ring kernels, the streaming
stacks, split-K at tree nodes, the simulated tensor-parallel partials and
their combine -- must then reproduce the oracle's tree exactly (TBIK
summary page, "technical framework": local reduction, then the binary tree;
IsoExec brief, section 叁: fixed blocking).  Leaf magnitudes span 2^-12..2^12
so different trees round differently (tests/test_exact_leaf_inputs.py shows
that on the CPU).

Shapes reach every launch path of tbik_gemm: the thin 16- and 32-row ring
tiles (K = 14336, M <= 32, K split into its 8 groups or tp = 4 / 8 shards),
the small-M kernel (other K, tp = 2), the narrow and wide ring tiles with
the perfect-tree, 4-, 8-, 11- and 28-leaf group schedules, paired shards
(tp = 8 at K = 14336 with many tiles), all shards of a tile in one
workgroup (one group per shard, 256 to 512 tiles), split-K at tree nodes, the
strided-batched kernel and the LM-head GEMM with fused row maxima.
"""
import os

import numpy as np
import pytest
import torch

import tp_invariant_numerics_amd as tb
from tp_invariant_numerics_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
MS = (1, 16, 17, 24, 32, 33, 100, 255, 256, 512)
KS = (1024, 2048, 4096, 5632, 14336)
N = 4112                       # 32 x 128 + 16: ragged in every tile width


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    tb.lib()


def _cols(n, seed):
    """Sampled output columns: every tile edge the kernels use, plus random."""
    edge = set()
    for w in (16, 32, 64, 128):
        for c in range(0, n, w):
            if c % 512 == 0 or c >= n - 2 * w:
                edge.update((c, c - 1, c + w - 1))
    rnd = np.random.default_rng(seed).choice(n, 48, replace=False)
    cols = sorted(c for c in edge | set(rnd.tolist()) | {n - 1} if 0 <= c < n)
    return np.array(cols, np.int64)


def _u32(t):
    return t.detach().cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("K", KS)
def test_mfma_exact_leaves_equal_oracle(orc, K):
    Mmax = max(MS)
    A = inputs.one_per_block_bf16((Mmax, K), 11000 + K, spread=12)
    W = inputs.normal_bf16((N, K), 11001 + K, device=DEV)
    cols = _cols(N, K)
    say("exact leaves: oracle", Mmax, len(cols), K)
    ref = orc.gemm(inputs.bits(A), inputs.bits(W[torch.from_numpy(cols).to(DEV)]))
    refb = ref.view(np.uint32)
    Ad = A.to(DEV)
    ci = torch.from_numpy(cols).to(DEV)
    for M in MS:
        for tp in (1, 2, 4, 8):
            variants = [("ws", lambda: tb.tbik_gemm(Ad[:M], W)[0]),
                        ("nows", lambda: tb.tbik_gemm(Ad[:M], W, ws=None)[0])] if tp == 1 else \
                       [("tpsim", lambda: tb.tbik_gemm_tpsim(Ad[:M], W, tp)[0])]
            for name, fn in variants:
                say("exact leaves", "M", M, "K", K, "tp", tp, name)
                got = _u32(fn().index_select(1, ci))
                bad = np.argwhere(got != refb[:M])
                assert bad.size == 0, ("M", M, "K", K, "tp", tp, name, "first mismatch",
                                       bad[0].tolist(), int(cols[bad[0][1]]))


@pytest.mark.parametrize("B,M,Nb,K", [(2, 40, 72, 1024), (3, 100, 130, 5632), (2, 17, 40, 2048)])
def test_mfma_exact_leaves_strided_batched(orc, B, M, Nb, K):
    A = inputs.one_per_block_bf16((B, M, K), 11100 + K, spread=12)
    W = inputs.normal_bf16((B, Nb, K), 11101 + K)
    say("exact leaves, strided batched", B, M, Nb, K)
    C, _ = tb.tbik_gemm_strided_batched(A.to(DEV), W.to(DEV))
    for b in range(B):
        ref = orc.gemm(inputs.bits(A[b]), inputs.bits(W[b]))
        assert np.array_equal(_u32(C[b]), ref.view(np.uint32)), b


def test_mfma_exact_leaves_lm_head(orc):
    """The LM-head shape (M = 512, K = 4096, N = 151936) through the GEMM with
    fused row maxima: sampled logits bit-exact against the oracle, the row
    maxima equal to the maximum of each 64-column block."""
    M, K, V = 512, 4096, 151936
    A = inputs.one_per_block_bf16((M, K), 11200, spread=12)
    W = inputs.normal_bf16((V, K), 11201, std=0.02, device=DEV)
    cols = np.unique(np.concatenate([_cols(V, 3)[:200], np.arange(V - 200, V),
                                     np.random.default_rng(4).choice(V, 200, replace=False)]))
    ci = torch.from_numpy(cols).to(DEV)
    say("exact leaves, lm head")
    ref = orc.gemm(inputs.bits(A), inputs.bits(W.index_select(0, ci)))
    logits, pmax = tb.tbik_gemm_logits(A.to(DEV), W)
    assert np.array_equal(_u32(logits.index_select(1, ci)), ref.view(np.uint32))
    nb = (V + 63) // 64
    pad = torch.full((M, nb * 64), -float("inf"), device=DEV)
    pad[:, :V] = logits
    assert torch.equal(pmax, pad.view(M, nb, 64).amax(dim=2))


def test_mfma_exact_leaves_golden_tree_probes():
    """The hand-derived 2^24 tree probes (tests/golden/tree_probes.txt) as
    GEMMs with exact leaves on the matrix cores, at batch sizes reaching the
    small-M and ring kernels; the expected value comes from the fixture."""
    path = os.path.join(os.path.dirname(__file__), "golden", "tree_probes.txt")
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        n, big, expected = (int(t) for t in line.split())
        K = 64 * n
        for M in (1, 40, 300):
            A = inputs.one_per_block_bf16((M, K), 11300 + n, value=1.0)
            A[:, big * 64:(big + 1) * 64] *= 2.0 ** 24
            W = torch.ones((130, K), dtype=torch.bfloat16, device=DEV)
            say("golden tree probe", n, big, "M", M)
            C, _ = tb.tbik_gemm(A.to(DEV), W)
            assert torch.all(C == float(expected)), (n, big, M, C.unique().tolist()[:4])


@pytest.mark.parametrize("K", (2048, 4096, 5632, 8192))
def test_mfma_exact_leaves_all_shards_per_workgroup(orc, K):
    """Shapes with 256 to 512 wide tiles and one tree group per shard (or
    11-leaf groups), where a workgroup streams every shard of its tile
    through one ring and writes each shard's node as it completes: K = 2048
    (tp 2, 4, 8 give shards of 16, 8 and 4 leaves), K = 4096 (32, 16, 8),
    K = 5632 (4, 2 or 1 groups of 11 leaves) and K = 8192 (tp 4: 32).  C and
    every shard partial are bit-exact against the oracle's simulated tensor
    parallelism on sampled rows and columns; the M = 4000 rows of A repeat
    the same 512 rows (the last copy cut short), so every row block is
    compared with the same oracle rows."""
    M, Nw = 4000, 1040                 # 32 x 9 = 288 tiles of 128 x 128, ragged M and N
    A512 = inputs.one_per_block_bf16((512, K), 11400 + K, spread=12)
    A = A512.repeat(8, 1)[:M]
    W = inputs.normal_bf16((Nw, K), 11401 + K, device=DEV)
    cols = _cols(Nw, K + 1)
    ci = torch.from_numpy(cols).to(DEV)
    rows = np.unique(np.concatenate([np.arange(0, 512, 37), [0, 127, 128, (M - 1) % 512, 511]]))
    Ad = A.to(DEV)
    for tp in ((2, 4, 8) if K < 8192 else (4,)):
        say("exact leaves, all shards per workgroup: K", K, "tp", tp)
        refC, refP = orc.gemm_tpsim(inputs.bits(A512[rows]),
                                    inputs.bits(W.index_select(0, ci)), tp)
        C, _, ws = tb.tbik_gemm_tpsim(Ad, W, tp)
        for blk in range((M + 511) // 512):
            keep = blk * 512 + rows < M              # the last block is ragged
            bi = torch.from_numpy(blk * 512 + rows[keep]).to(DEV)
            got = _u32(C.index_select(0, bi).index_select(1, ci))
            assert np.array_equal(got, refC.view(np.uint32)[keep]), ("C", K, tp, blk)
            for t in range(tp):
                got = _u32(ws[t].index_select(0, bi).index_select(1, ci))
                assert np.array_equal(got, refP[t].view(np.uint32)[keep]), ("partial", K, tp, t)
