"""CPU checks of the exact-leaf inputs used by the GPU bit-parity tests of the
matrix-core GEMM.

A row with one nonzero entry per 64-wide K block, multiplied by a dense
operand, gives every 64-wide leaf a single nonzero product.  bf16 x bf16
products are exact in fp32 (rounding-alignment article, "the problem": 7
stored mantissa bits), and adding zeros to one value is exact, so such a
leaf has the same bits whatever order a matrix unit adds its 64 products
in.  The tree above the leaves is then the only thing that decides the
result -- which these checks show is visible in the bits: the oracle's
GEMM equals its TREE over the explicit single-product leaves, and other
plausible trees (sequential, flat pairwise, groups swapped for PAIR's carry
rule) give different bits on many outputs.
"""
import numpy as np
import pytest
import torch

from tp_invariant_numerics_amd import inputs


def _seq(v):
    s = np.float32(0)
    for x in v:
        s = np.float32(s + x)
    return s


def _flat_pairwise(v):
    v = list(np.asarray(v, np.float32))
    while len(v) > 1:
        nxt = [np.float32(v[i] + v[i + 1]) for i in range(0, len(v) - 1, 2)]
        if len(v) % 2:
            nxt.append(v[-1])
        v = nxt
    return v[0]


def _pair_carry_first(v):
    """PAIR with the odd element carried at the front instead of the end."""
    v = list(np.asarray(v, np.float32))
    while len(v) > 1:
        if len(v) % 2:
            v = [v[0]] + [np.float32(v[i] + v[i + 1]) for i in range(1, len(v) - 1, 2)]
        else:
            v = [np.float32(v[i] + v[i + 1]) for i in range(0, len(v), 2)]
    return v[0]


def _tree_variant(leaves, T, inner):
    G = len(leaves) // T
    groups = [inner(leaves[g * G:(g + 1) * G]) for g in range(T)]
    return _flat_pairwise(groups)


@pytest.mark.parametrize("K", [1024, 5632, 14336])
def test_exact_leaf_gemm_is_the_tree_of_single_products(orc, K):
    M, N = 6, 5
    A = inputs.bits(inputs.one_per_block_bf16((M, K), 10 + K))
    W = inputs.bits(inputs.normal_bf16((N, K), 20 + K))
    a = orc.bf16_to_f32(A)
    w = orc.bf16_to_f32(W)
    assert np.all((a.reshape(M, -1, 64) != 0).sum(-1) == 1)
    C = orc.gemm(A, W)
    nb = K // 64
    T = orc.tree_T(nb)
    differ = {"seq": 0, "flat": 0, "carry_first": 0}
    for i in range(M):
        k = np.nonzero(a[i])[0]
        for j in range(N):
            leaves = (a[i, k] * w[j, k]).astype(np.float32)     # exact products
            assert np.float32(orc.tree(leaves)).view(np.uint32) == C[i, j].view(np.uint32)
            differ["seq"] += _seq(leaves).view(np.uint32) != C[i, j].view(np.uint32)
            differ["flat"] += _flat_pairwise(leaves).view(np.uint32) != C[i, j].view(np.uint32)
            differ["carry_first"] += (_tree_variant(leaves, T, _pair_carry_first).view(np.uint32)
                                      != C[i, j].view(np.uint32))
    # a wrong tree is seen on a good share of the outputs (the flat pairwise
    # tree and the carry rule coincide with the definition when every level
    # is even, i.e. for power-of-two groups)
    assert differ["seq"] >= M * N // 3, differ
    if (nb // T) & (nb // T - 1):
        assert differ["flat"] >= M * N // 4, differ
        assert differ["carry_first"] >= M * N // 4, differ


def test_golden_tree_probe_as_gemm(orc):
    """The 2^24-scaled tree probes (tests/golden/tree_probes.txt) written as a
    GEMM with exact leaves: ones at one position per 64-wide block, 2^24 in
    the probe's block, against a row of ones."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tree_probes.txt")
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        n, big, expected = (int(t) for t in line.split())
        A = inputs.one_per_block_bf16((1, 64 * n), 7 + n, value=1.0)
        A[0, big * 64:(big + 1) * 64] *= 2.0 ** 24
        W = torch.ones((1, 64 * n), dtype=torch.bfloat16)
        C = orc.gemm(inputs.bits(A), inputs.bits(W))
        assert C[0, 0] == np.float32(expected), (n, big, float(C[0, 0]))
