"""CPU checks of the C ABI boundary (no kernel is launched here).

* every function declared in include/tbik.h is exported by libtbik.so;
* invalid arguments are rejected on the host with the documented code
  (every case below fails validation, so no device pointer is touched);
* the host RoPE-table helper equals the oracle's table bit for bit.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, E_NULL, E_SHAPE, E_TP, E_ALIGN, E_WS, E_LAUNCH, E_ARG = 0, -1, -2, -3, -4, -5, -6, -7

FAKE = C.c_void_p(1 << 20)        # aligned, never dereferenced (validation fails first)
FAKE2 = C.c_void_p(2 << 20)
FAKE3 = C.c_void_p(3 << 20)
MISAL = C.c_void_p((1 << 20) + 1)     # violates every element alignment


@pytest.fixture(scope="module")
def L():
    import tp_invariant_numerics_amd as t
    return t.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "tbik.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tbik_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("tbik_gemm", "tbik_gemm_tpsim", "tbik_rmsnorm_residual", "tbik_logsoftmax_gather",
              "tbik_rope", "tbik_swiglu"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_every_declared_symbol_has_a_binding_signature(L):
    """Each entry point has explicit ctypes argument types: without them a
    64-bit device pointer would be passed as a C int and truncated."""
    import tp_invariant_numerics_amd as t
    sigs = t._sigs()
    for name in declared_functions():
        assert name in sigs, name
        assert getattr(L, name).argtypes is not None, name


def test_gather_rows_validation(L):
    g = L.tbik_gather_rows
    assert g(None, 8, 4, FAKE, 2, 8, FAKE2, 8, None) == E_NULL
    assert g(FAKE, 4, 4, FAKE2, 2, 8, FAKE3, 8, None) == E_SHAPE      # ld_table < cols
    assert g(FAKE, 8, 4, FAKE2, 2, 8, FAKE3, 4, None) == E_SHAPE      # ld_out < cols
    assert g(FAKE, 8, -1, FAKE2, 2, 8, FAKE3, 8, None) == E_SHAPE
    assert g(MISAL, 8, 4, FAKE2, 2, 8, FAKE3, 8, None) == E_ALIGN
    assert g(FAKE, 8, 4, FAKE2, 0, 8, FAKE3, 8, None) == OK           # nothing to copy


def test_logprob_fused_validation(L):
    g = L.tbik_gemm_logits
    assert g(FAKE, 64, FAKE2, 64, None, 64, 4, 4, 64, FAKE3, 1, None) == E_NULL
    assert g(FAKE, 64, FAKE2, 64, FAKE3, 64, 4, 4, 64, None, 1, None) == E_NULL
    assert g(FAKE, 64, FAKE2, 64, FAKE3, 128, 4, 128, 64, FAKE, 1, None) == E_SHAPE  # ld_pmax
    assert g(FAKE, 64, FAKE2, 64, FAKE3, 64, 4, 4, 64, MISAL, 1, None) == E_ALIGN
    assert g(FAKE, 64, FAKE2, 64, FAKE3, 64, 0, 4, 64, FAKE, 1, None) == OK
    h = L.tbik_logsoftmax_gather_pmax
    assert h(FAKE, 8, FAKE2, FAKE3, 4, 8, 1, None, 1, 1, FAKE, 1 << 20, None) == E_NULL
    assert h(FAKE, 8, FAKE2, FAKE3, 4, 8, 1, FAKE, 0, 1, FAKE, 1 << 20, None) == E_SHAPE
    assert h(FAKE, 8, FAKE2, FAKE3, 4, 8, 3, FAKE, 1, 1, FAKE, 1 << 20, None) == E_TP
    assert h(FAKE, 8, FAKE2, FAKE3, 4, 8, 1, FAKE, 1, 1, None, 0, None) == E_WS


def test_attention_validation(L):
    a = L.tbik_attention_causal
    sc = C.c_float(0.088)
    assert a(None, 256, FAKE, 256, FAKE2, 512, FAKE3, 256, 512, 2, 128, 1, sc, None) == E_NULL
    assert a(FAKE, 256, FAKE, 256, FAKE2, 512, FAKE3, 256, 512, 2, 64, 1, sc, None) == E_SHAPE
    assert a(FAKE, 256, FAKE, 256, FAKE2, 512, FAKE3, 256, 500, 2, 128, 1, sc, None) == E_SHAPE
    assert a(FAKE, 128, FAKE, 256, FAKE2, 512, FAKE3, 256, 512, 2, 128, 1, sc, None) == E_SHAPE
    assert a(FAKE, 256, FAKE, 256, FAKE2, 256, FAKE3, 256, 512, 2, 128, 1, sc, None) == E_SHAPE
    assert a(MISAL, 256, FAKE, 256, FAKE2, 512, FAKE3, 256, 512, 2, 128, 1, sc, None) == E_ALIGN
    assert a(FAKE, 256, FAKE, 256, FAKE2, 512, FAKE3, 256, 512, 2, 128, 0, sc, None) == OK


def test_version_and_strerror(L):
    import tp_invariant_numerics_amd as t
    assert t.tbik_version() >= 10000
    for code in (OK, E_NULL, E_SHAPE, E_TP, E_ALIGN, E_WS, E_LAUNCH, E_ARG, 17):
        assert isinstance(t.tbik_strerror(code), str) and t.tbik_strerror(code)


def test_tree_groups(L):
    assert [L.tbik_tree_groups(n) for n in (0, 1, 3, 6, 12, 28, 224, 151936)] == \
        [0, 1, 1, 2, 4, 4, 8, 8]


def test_gemm_validation(L):
    g = L.tbik_gemm
    # A NULL / W NULL / both outputs NULL
    assert g(None, 64, FAKE, 64, FAKE2, 64, None, 4, 4, 64, 0, None, 0, None) == E_NULL
    assert g(FAKE, 64, None, 64, FAKE2, 64, None, 4, 4, 64, 0, None, 0, None) == E_NULL
    assert g(FAKE, 64, FAKE2, 64, None, 64, None, 4, 4, 64, 0, None, 0, None) == E_NULL
    # K not a positive multiple of 64, negative sizes, small leading dims
    assert g(FAKE, 128, FAKE2, 128, FAKE3, 64, None, 4, 4, 100, 0, None, 0, None) == E_SHAPE
    assert g(FAKE, 64, FAKE2, 64, FAKE3, 64, None, 4, 4, 0, 0, None, 0, None) == E_SHAPE
    assert g(FAKE, 64, FAKE2, 64, FAKE3, 64, None, -1, 4, 64, 0, None, 0, None) == E_SHAPE
    assert g(FAKE, 32, FAKE2, 64, FAKE3, 64, None, 4, 4, 64, 0, None, 0, None) == E_SHAPE
    assert g(FAKE, 64, FAKE2, 64, FAKE3, 8, None, 4, 16, 64, 0, None, 0, None) == E_SHAPE
    # alignment: misaligned pointer, leading dimension not a multiple of 8
    assert g(MISAL, 64, FAKE2, 64, FAKE3, 64, None, 4, 4, 64, 0, None, 0, None) == E_ALIGN
    assert g(FAKE, 68, FAKE2, 64, FAKE3, 64, None, 4, 4, 64, 0, None, 0, None) == E_ALIGN
    assert g(FAKE, 64, FAKE2, 64, FAKE3, 3, None, 4, 4, 64, 0, None, 0, None) == E_SHAPE
    assert g(FAKE, 64, FAKE2, 64, MISAL, 64, None, 4, 4, 64, 0, None, 0, None) == E_ALIGN
    # leaf mode
    assert g(FAKE, 64, FAKE2, 64, FAKE3, 64, None, 4, 4, 64, 7, None, 0, None) == E_ARG
    # tree groups beyond the supported depth (K = 64 * 1031, a prime leaf count)
    assert g(FAKE, 66000, FAKE2, 66000, FAKE3, 64, None, 1, 1, 64 * 1031, 0, None, 0, None) == E_SHAPE


def test_gemm_tpsim_validation(L):
    g = L.tbik_gemm_tpsim
    # tp not in {1,2,4,8}; tp not dividing T (K = 64*28 has T = 4)
    assert g(FAKE, 64, FAKE2, 64, FAKE3, 64, None, 4, 4, 64, 3, 0, FAKE, 1 << 20, None) == E_TP
    assert g(FAKE, 1792, FAKE2, 1792, FAKE3, 64, None, 4, 4, 1792, 8, 0, FAKE, 1 << 20,
             None) == E_TP
    # workspace missing / too small
    assert g(FAKE, 1024, FAKE2, 1024, FAKE3, 64, None, 4, 4, 1024, 2, 0, None, 0,
             None) == E_WS
    need = L.tbik_gemm_tpsim_workspace_bytes(4, 4, 1024, 2)
    assert need == 2 * 4 * 4 * 4
    assert g(FAKE, 1024, FAKE2, 1024, FAKE3, 64, None, 4, 4, 1024, 2, 0, FAKE, need - 1,
             None) == E_WS


def test_gemm_workspace_split_policy(L):
    """K = 14336 (8 groups of 28 leaves): small M splits K into its 8 groups
    (thin tiles read only their group's K slice of A); M = 256 into the
    fewest parts that give every CU a 128 x 128 tile; scalar leaves, batched
    calls and K without 28-leaf groups never split."""
    ws = L.tbik_gemm_workspace_bytes
    for M in (1, 16, 17, 32):
        assert ws(M, 4096, 14336) == 8 * M * 4096 * 4, M
    assert ws(256, 4096, 14336) == 4 * 256 * 4096 * 4
    assert ws(32, 4096, 4096) == 0


def test_gemm_swiglu_validation(L):
    g = L.tbik_gemm_swiglu
    # F not a multiple of 16; H missing; M <= 32 (no fused kernel: nothing launched)
    assert g(FAKE, 1024, FAKE2, 1024, FAKE3, 24, 64, 24, 1024, 0, None) == E_SHAPE
    assert g(FAKE, 1024, FAKE2, 1024, None, 32, 64, 32, 1024, 0, None) == E_NULL
    assert g(FAKE, 1024, FAKE2, 1024, FAKE3, 32, 32, 32, 1024, 0, None) == E_SHAPE
    assert g(FAKE, 1024, FAKE2, 1024, FAKE3, 32, 64, 32, 1024, 7, None) == E_ARG


def test_combine_validation(L):
    assert L.tbik_tree_combine(None, 2, FAKE, 8, None, 1, 8, None) == E_NULL
    assert L.tbik_tree_combine(FAKE, 3, FAKE2, 8, None, 1, 8, None) == E_TP
    assert L.tbik_tree_combine(FAKE, 2, FAKE2, 4, None, 1, 8, None) == E_SHAPE


def test_rowop_validation(L):
    r = L.tbik_rmsnorm_residual
    assert r(None, FAKE, FAKE, FAKE, None, 1, 64, 64, 1e-6, None) == E_NULL
    assert r(FAKE, FAKE, FAKE, FAKE2, None, 1, 0, 64, 1e-6, None) == E_SHAPE
    assert r(FAKE, FAKE, FAKE, FAKE2, None, 1, 64, 32, 1e-6, None) == E_SHAPE
    assert r(FAKE, FAKE, FAKE, FAKE2, None, 1, 64, 64, -1.0, None) == E_ARG
    assert r(FAKE, FAKE, FAKE, MISAL, None, 1, 64, 64, 1e-6, None) == E_ALIGN
    assert r(FAKE, FAKE, FAKE, FAKE2, None, 1, 65537, 65537, 1e-6, None) == E_SHAPE
    # (every H in 1..65536 is accepted; odd group sizes such as 65534 =
    # 2 x 32767 are checked against the oracle on the GPU)
    ro = L.tbik_rope
    assert ro(FAKE, FAKE, None, FAKE, FAKE, 1, 1, 128, 128, 16, None) == E_NULL
    assert ro(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 130, 136, 16, None) == E_SHAPE
    assert ro(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 128, 128, 16, None) == E_SHAPE
    sw = L.tbik_swiglu
    assert sw(FAKE, None, FAKE, 1, 8, 8, 8, 8, None) == E_NULL
    assert sw(FAKE, FAKE, FAKE, 1, 16, 8, 16, 16, None) == E_SHAPE
    assert sw(FAKE, FAKE, MISAL, 1, 8, 8, 8, 8, None) == E_ALIGN
    # rounding location: only TBIK_ROUND_ONCE (0) and TBIK_ROUND_EACH_OP (1)
    assert L.tbik_rmsnorm_residual_ex(FAKE, FAKE, FAKE, FAKE2, None, 1, 64, 64, 1e-6, 2,
                                      None) == E_ARG
    assert L.tbik_rope_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 128, 16, -1, None) == E_ARG
    assert L.tbik_swiglu_ex(FAKE, FAKE, FAKE2, 1, 8, 8, 8, 8, 7, None) == E_ARG
    assert L.tbik_swiglu_ex(FAKE, None, FAKE, 1, 8, 8, 8, 8, 1, None) == E_NULL
    assert L.tbik_rmsnorm_residual_ex(FAKE, FAKE, FAKE, FAKE2, None, 0, 64, 64, 1e-6, 1,
                                      None) == OK
    ls = L.tbik_logsoftmax_gather
    assert ls(FAKE, 8, FAKE, FAKE, 2, 8, 3, FAKE, 1 << 20, None) == E_TP
    # a row stages T * ceil(G / 16) chunk sums in LDS: with V = 655105 (odd,
    # one group) that is 40945 values, more than fit beside the kernel's own
    # 64 bytes (refused by the launcher before it launches anything)
    assert ls(FAKE, 655105, FAKE, FAKE, 1, 655105, 1, FAKE, 1 << 20, None) == E_SHAPE
    assert ls(FAKE, 24, FAKE, FAKE, 2, 12, 8, FAKE, 1 << 20, None) == E_TP   # T(12) = 4
    assert ls(FAKE, 8, FAKE, FAKE, 2, 8, 1, None, 0, None) == E_WS
    assert ls(FAKE, 8, FAKE, FAKE, 2, 8, 1, FAKE, 4, None) == E_WS
    sc = L.tbik_softmax_causal
    assert sc(FAKE, 64, 0, FAKE2, 64, 0, 4, 64, 1, -1, 1.0, None) == E_SHAPE
    assert sc(FAKE, 64, 0, FAKE2, 64, 0, 4, 64, 1, 0, float("inf"), None) == E_ARG
    assert L.tbik_primitive(9, FAKE, FAKE2, 4, None) == E_ARG
    assert L.tbik_primitive(0, None, FAKE2, 4, None) == E_NULL


def test_training_validation(L):
    # transpose
    assert L.tbik_transpose_bf16(None, 8, FAKE2, 8, 4, 8, None) == E_NULL
    assert L.tbik_transpose_bf16(FAKE, 4, FAKE2, 8, 4, 8, None) == E_SHAPE
    assert L.tbik_transpose_bf16(FAKE, 8, FAKE2, 8, 0, 8, None) == OK
    # input gradient: the reduced dimension N must be a multiple of 64
    dg = L.tbik_gemm_dgrad
    assert dg(FAKE, 96, FAKE2, 64, FAKE3, 64, None, 4, 96, 64, 0, FAKE, 1 << 20, None) == E_SHAPE
    assert dg(FAKE, 128, FAKE2, 64, FAKE3, 64, None, 4, 128, 64, 0, None, 0, None) == E_WS
    assert dg(FAKE, 128, FAKE2, 64, FAKE3, 64, None, 4, 128, 64, 0, FAKE, 64, None) == E_WS
    assert dg(FAKE, 128, FAKE2, 64, FAKE3, 64, None, 0, 128, 64, 0, None, 0, None) == OK
    # weight gradient: tokens a multiple of 64, dp dividing T(M/64)
    wg = L.tbik_gemm_wgrad
    assert wg(FAKE, 64, FAKE2, 64, FAKE3, 64, 100, 64, 64, 1, 0, FAKE, 1 << 20, None) == E_SHAPE
    assert wg(FAKE, 64, FAKE2, 64, FAKE3, 64, 256, 64, 64, 3, 0, FAKE, 1 << 20, None) == E_TP
    assert wg(FAKE, 64, FAKE2, 64, FAKE3, 64, 64 * 12, 64, 64, 8, 0, FAKE, 1 << 24, None) == E_TP
    assert wg(FAKE, 64, FAKE2, 64, FAKE3, 64, 256, 64, 64, 2, 0, FAKE, 1024, None) == E_WS
    assert L.tbik_gemm_wgrad_workspace_bytes(256, 64, 32, 2) == 32768 + 16384 + 2 * 64 * 32 * 4
    # backward passes
    assert L.tbik_rope_backward(FAKE, FAKE, None, FAKE, FAKE, 1, 1, 128, 128, 16, None) == E_NULL
    sb = L.tbik_swiglu_backward
    assert sb(FAKE, FAKE, FAKE, FAKE2, None, 1, 8, 8, 8, 8, 8, 8, None) == E_NULL
    assert sb(FAKE, FAKE, FAKE, FAKE2, FAKE3, 1, 16, 16, 16, 8, 16, 16, None) == E_SHAPE
    rb = L.tbik_rmsnorm_backward
    assert rb(FAKE, FAKE, FAKE, FAKE, None, FAKE2, FAKE3, 100, 64, 64, 1e-6, 1, FAKE, 1 << 20,
              None) == E_SHAPE
    assert rb(FAKE, FAKE, FAKE, FAKE, None, FAKE2, FAKE3, 128, 64, 64, 1e-6, 4, FAKE, 1 << 20,
              None) == E_TP
    assert rb(FAKE, FAKE, FAKE, FAKE, None, FAKE2, None, 7, 64, 64, 1e-6, 1, None, 0,
              None) == E_WS
    assert rb(FAKE, FAKE, FAKE, FAKE, None, FAKE2, None, 0, 64, 64, 1e-6, 1, None, 0,
              None) == OK


def test_empty_shapes_are_no_ops(L):
    # M = 0 / rows = 0 return OK before touching any pointer or launching
    assert L.tbik_gemm(FAKE, 64, FAKE2, 64, FAKE3, 64, None, 0, 4, 64, 0, None, 0, None) == OK
    assert L.tbik_rmsnorm_residual(FAKE, FAKE, FAKE, FAKE2, None, 0, 64, 64, 1e-6, None) == OK
    assert L.tbik_swiglu(FAKE, FAKE, FAKE2, 0, 8, 8, 8, 8, None) == OK
    assert L.tbik_primitive(0, FAKE, FAKE2, 0, None) == OK


def test_rope_table_equals_oracle(orc):
    import tp_invariant_numerics_amd as t
    for theta, d, maxp in ((1e6, 128, 32768), (1e4, 64, 4096), (500000.0, 16, 100)):
        c, s = t.tbik_rope_table(theta, d, maxp)
        oc, os_ = orc.rope_table(theta, d, maxp)
        assert np.array_equal(c.numpy().view(np.uint32), oc.view(np.uint32))
        assert np.array_equal(s.numpy().view(np.uint32), os_.view(np.uint32))


def test_gemm_noalloc_validation(L):
    """The allocation-free GEMM validates like tbik_gemm and refuses, before
    any launch, shapes whose split-K partials exceed its scratch array."""
    g = L.tbik_gemm_noalloc
    assert L.tbik_gemm_noalloc_max_bytes() == 16 << 20
    assert g(None, 64, FAKE, 64, FAKE2, 64, None, 1, 1, 64, 0, None) == E_NULL
    assert g(FAKE, 64, FAKE, 64, FAKE2, 64, None, 1, 1, 65, 0, None) == E_SHAPE
    assert g(MISAL, 64, FAKE, 64, FAKE2, 64, None, 1, 1, 64, 0, None) == E_ALIGN
    assert g(FAKE, 64, FAKE, 64, FAKE2, 64, None, 1, 1, 64, 7, None) == E_ARG
    # M = 256, N = 16384, K = 14336 splits into two tree nodes: 32 MiB of partials
    assert L.tbik_gemm_workspace_bytes(256, 16384, 14336) > (16 << 20)
    assert g(FAKE, 14336, FAKE, 14336, FAKE2, 16384, None, 256, 16384, 14336, 0, None) == E_WS
    assert g(FAKE, 64, FAKE, 64, FAKE2, 64, None, 0, 5, 64, 0, None) == OK   # empty: no-op


def test_microbench_validation(L):
    """The ceiling microbenchmarks validate on the host like every other entry
    point (each case below fails before any launch)."""
    assert L.tbik_bench_mfma_flops(0, 5) == 0
    assert L.tbik_bench_mfma_flops(2, 3) == 2 * 8 * 8 * 3 * 16384
    assert L.tbik_bench_mfma(None, FAKE, 1, 1, None) == E_NULL
    assert L.tbik_bench_mfma(FAKE, FAKE2, 0, 1, None) == E_SHAPE
    assert L.tbik_bench_mfma(MISAL, FAKE2, 1, 1, None) == E_ALIGN
    assert L.tbik_bench_hbm_read(FAKE, 100, FAKE2, 1, None) == E_SHAPE      # not a multiple of 16
    assert L.tbik_bench_hbm_read(MISAL, 1024, FAKE2, 1, None) == E_ALIGN
    assert L.tbik_bench_hbm_copy(FAKE, None, 1024, 1, None) == E_NULL
    assert L.tbik_bench_hbm_copy(FAKE, FAKE2, 1024, 0, None) == E_SHAPE
    cl = L.tbik_bench_copy_lds
    assert cl(None, 32768, 1, FAKE2, 1, None) == E_NULL
    assert cl(FAKE, 32768 + 16, 1, FAKE2, 1, None) == E_SHAPE               # not whole stages
    assert cl(FAKE, 16384, 1, FAKE2, 1, None) == E_SHAPE                    # below one stage
    assert cl(FAKE, 1 << 31, 1, FAKE2, 1, None) == E_SHAPE                  # beyond the 32-bit range
    assert cl(FAKE, 32768, 0, FAKE2, 1, None) == E_SHAPE
    assert cl(FAKE, 32768, 1, FAKE2, 0, None) == E_SHAPE
    assert cl(MISAL, 32768, 1, FAKE2, 1, None) == E_ALIGN
