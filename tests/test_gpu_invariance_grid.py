"""The invariance grid the method promises, at the workloads' full sizes.

TBIK summary page, Abstract: outputs must not change with the TP size or the
batch size.  Checked bit for bit, stopping at the first mismatch:

- the row-parallel down projection (K = 14336, N = 4096, A ~N(0,1),
  W ~N(0,0.02)): every batch size M in 1..256 at every simulated TP size in
  {2, 4, 8}, against the rows of the M = 256, tp = 1 product (tp = 1 over
  the same M range is in the parity suite);
- the LM-head logprob path (M = 512, K = 4096, V = 151936, uniform targets):
  logits, their fused row maxima and the logprobs of a sub-batch equal the
  corresponding rows of the full batch, for tp 1 and 4.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    tb.lib()


def _i32(t):
    return t.view(torch.int32)


def test_downproj_tp_by_batch_grid():
    K, N, Mmax = 14336, 4096, 256
    A = inputs.normal_bf16((Mmax, K), 13000, device=DEV)
    W = inputs.normal_bf16((N, K), 13001, std=0.02, device=DEV)
    ref = _i32(tb.tbik_gemm(A, W)[0])
    ws_all = torch.empty((8 * Mmax * N,), dtype=torch.float32, device=DEV)
    out_all = torch.empty((Mmax * N,), dtype=torch.float32, device=DEV)
    checked = 0
    for tp in (2, 4, 8):
        say("grid tp", tp, "M 1..256")
        for M in range(1, Mmax + 1):
            ws = ws_all[:tp * M * N].view(tp, M, N)
            out = out_all[:M * N].view(M, N)
            tb.tbik_gemm_tpsim(A[:M], W, tp, ws=ws, out=out)
            if not torch.equal(_i32(out), ref[:M]):
                bad = (_i32(out) != ref[:M]).nonzero()[0].tolist()
                pytest.fail("tp %d, M %d: first mismatch at %s" % (tp, M, bad))
            checked += 1
    say("grid: %d (tp, M) cases bitwise equal" % checked)
    assert checked == 3 * Mmax


@pytest.fixture(scope="module")
def lm_head():
    M, K, V = 512, 4096, 151936
    A = inputs.normal_bf16((M, K), 13100, device=DEV)
    W = inputs.normal_bf16((V, K), 13101, std=0.02, device=DEV)
    tgt = inputs.uniform_int(M, V, 13102, device=DEV)
    logits, pmax = tb.tbik_gemm_logits(A, W)
    lps = {tp: tb.tbik_logsoftmax_gather_pmax(logits, tgt, pmax, tp)[0] for tp in (1, 4)}
    return A, W, tgt, logits, pmax, lps


def test_lm_head_logprobs_tp1_equals_tp4(lm_head):
    *_, lps = lm_head
    assert torch.equal(_i32(lps[1]), _i32(lps[4]))
    assert torch.isfinite(lps[1]).all()


@pytest.mark.parametrize("lo,M", [(0, 1), (0, 2), (5, 17), (100, 64), (0, 255), (256, 256),
                                  (511, 1), (1, 511)])
def test_lm_head_sub_batch_equals_full_batch(lm_head, lo, M):
    A, W, tgt, logits, pmax, lps = lm_head
    say("lm head sub-batch", lo, M)
    lg, pm = tb.tbik_gemm_logits(A[lo:lo + M], W)
    assert torch.equal(_i32(lg), _i32(logits[lo:lo + M]))
    assert torch.equal(_i32(pm), _i32(pmax[lo:lo + M]))
    for tp in (1, 4):
        lp, _ = tb.tbik_logsoftmax_gather_pmax(lg, tgt[lo:lo + M], pm, tp)
        assert torch.equal(_i32(lp), _i32(lps[tp][lo:lo + M])), tp
        # the standalone log-softmax (its own row maxima) gives the same bits
        lp2, _ = tb.tbik_logsoftmax_gather(lg, tgt[lo:lo + M], tp)
        assert torch.equal(_i32(lp2), _i32(lp)), tp
