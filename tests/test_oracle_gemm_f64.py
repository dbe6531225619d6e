"""Pins of the oracle's binary64 GEMM (``or_gemm_f64``).

The binary64 product is the reference of every accuracy gate on the MFMA
GEMM (normwise error and the elementwise summation bound), so it is pinned
here against things that do not come from it:

- exact integer arithmetic: on data whose products and partial sums are all
  multiples of one power of two below 2^53, every binary64 summation order
  is exact, so the result must equal the integer dot product exactly;
- the correctly rounded exact sum (``math.fsum`` of the exact products):
  a sequential binary64 sum of n terms lies within gamma_{n-1} * sum|p| of
  it, with the binary64 unit roundoff 2^-53 (Higham, Accuracy and Stability
  of Numerical Algorithms, recursive summation);
- strided operands and output (row strides larger than the row length);
- planted mistakes on the CPU: a binary32 accumulation, a transposed
  operand and a dropped term each break the bound, so the checks can see
  them.
"""
import ctypes as C
import math

import numpy as np
import pytest
import torch

from tp_invariant_numerics_amd import inputs

U64 = 2.0 ** -53


def gamma64(n):
    return n * U64 / (1 - n * U64)


def _dec(orc, b):
    return orc.bf16_to_f32(b).astype(np.float64)


def _exact_fsum(a, w):
    """Correctly rounded sum of the exact products, one output at a time."""
    M, N = a.shape[0], w.shape[0]
    return np.array([[math.fsum(a[i] * w[j]) for j in range(N)] for i in range(M)])


def _scaled_ints(shape, seed):
    """bf16 values k * 2^e, k integer in [-255, 255], e in [-3, 3]: exactly
    representable (8 significant bits).  Returns (bits, k * 2^(e+3) as int64)."""
    g = np.random.default_rng(seed)
    k = g.integers(-255, 256, shape)
    e = g.integers(-3, 4, shape)
    v = (k * np.exp2(e)).astype(np.float32)
    b = inputs.bits(torch.from_numpy(v).to(torch.bfloat16))
    return b, (k * (1 << 3) * np.exp2(e)).astype(np.int64)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 64), (4, 7, 100), (2, 9, 2048), (6, 3, 517)])
def test_gemm_f64_exact_on_scaled_integers(orc, M, N, K):
    # products are multiples of 2^-6 below 2^22; K <= 2048 terms keep every
    # partial sum a multiple of 2^-6 below 2^33: exact in binary64
    A, ai = _scaled_ints((M, K), 100 + K)
    W, wi = _scaled_ints((N, K), 200 + K)
    got = orc.gemm_f64(A, W)
    exact = (ai @ wi.T).astype(np.float64) / 64.0
    assert np.array_equal(got, exact)


@pytest.mark.parametrize("M,N,K", [(3, 4, 64), (5, 2, 333), (2, 6, 1792), (7, 1, 4096)])
def test_gemm_f64_within_binary64_bound_of_exact_sum(orc, M, N, K):
    A = inputs.bits(inputs.normal_bf16((M, K), 300 + K))
    W = inputs.bits(inputs.normal_bf16((N, K), 400 + K, std=0.02))
    a, w = _dec(orc, A), _dec(orc, W)
    got = orc.gemm_f64(A, W)
    exact = _exact_fsum(a, w)
    bound = gamma64(max(K - 1, 1)) * (np.abs(a) @ np.abs(w).T) + 2 * U64 * np.abs(exact)
    assert np.all(np.abs(got - exact) <= bound)
    # and well inside binary32 resolution: the reference of a 1e-5 gate
    assert np.max(np.abs(got - exact)) <= 1e-13 * np.max(np.abs(a) @ np.abs(w).T)


def test_gemm_f64_strided_operands_and_output(orc):
    # the C entry point with row strides beyond the row lengths
    M, N, K = 5, 7, 192
    lda, ldw, ldc = K + 13, K + 64, N + 5
    A = inputs.bits(inputs.normal_bf16((M, lda), 501))
    W = inputs.bits(inputs.normal_bf16((N, ldw), 502))
    out = np.full((M, ldc), 7.5, np.float64)
    lib = orc.lib()
    p = lambda x: x.ctypes.data_as(C.c_void_p)  # noqa: E731
    rc = lib.or_gemm_f64(p(A), lda, p(W), ldw, p(out), ldc, M, N, K, 2)
    assert rc == 0
    ref = orc.gemm_f64(np.ascontiguousarray(A[:, :K]), np.ascontiguousarray(W[:, :K]))
    assert np.array_equal(out[:, :N], ref)
    assert np.all(out[:, N:] == 7.5)              # padding untouched
    exact = _exact_fsum(_dec(orc, A[:, :K]), _dec(orc, W[:, :K]))
    assert np.max(np.abs(out[:, :N] - exact)) <= 1e-13 * np.max(np.abs(exact))


def test_gemm_f64_planted_mistakes_are_caught(orc):
    """Mistakes planted in CPU copies of the binary64 reference (never in the
    library): each violates the bound the real function meets."""
    M, N, K = 4, 5, 4096
    A = inputs.bits(inputs.normal_bf16((M, K), 601))
    W = inputs.bits(inputs.normal_bf16((N, K), 602))
    a, w = _dec(orc, A), _dec(orc, W)
    exact = _exact_fsum(a, w)
    bound = gamma64(K - 1) * (np.abs(a) @ np.abs(w).T) + 2 * U64 * np.abs(exact)
    assert np.all(np.abs(orc.gemm_f64(A, W) - exact) <= bound)

    # (1) binary32 accumulation of the same exact products
    f32 = np.zeros((M, N), np.float32)
    for k in range(K):
        f32 = (f32 + np.outer(a[:, k], w[:, k]).astype(np.float32)).astype(np.float32)
    assert np.any(np.abs(f32.astype(np.float64) - exact) > bound)
    # (2) a transposed operand (W read as [K, N] on a square problem)
    sq = inputs.bits(inputs.normal_bf16((64, 64), 603))
    s = _dec(orc, sq)
    ex_sq = _exact_fsum(s, s)
    wrong = s @ s                                  # A W instead of A W^T
    bsq = gamma64(63) * (np.abs(s) @ np.abs(s).T) + 2 * U64 * np.abs(ex_sq)
    assert np.array_equal(np.abs(orc.gemm_f64(sq, sq) - ex_sq) <= bsq, np.ones_like(bsq, bool))
    assert np.any(np.abs(wrong - ex_sq) > bsq)
    # (3) a dropped last term
    dropped = a[:, :K - 1] @ w[:, :K - 1].T
    assert np.any(np.abs(dropped - exact) > bound)
