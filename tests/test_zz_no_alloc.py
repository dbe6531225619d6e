"""tbik_gemm_noalloc (the GEMM with its split-K partials in the library's own
device scratch, for callers that cannot allocate) against tbik_gemm with a
caller workspace: bit for bit, on consecutive calls that reuse the scratch,
the second with a smaller input."""
import numpy as np
import pytest
import torch

import tp_invariant_numerics_amd as tb
from tp_invariant_numerics_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def _u32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def test_gemm_noalloc_equals_gemm_with_workspace():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    tb.lib()
    cap = tb.lib().tbik_gemm_noalloc_max_bytes()
    assert cap == 16 << 20
    # the down projection's batch sizes (split into tree nodes) then a
    # smaller, ragged call that reuses the same scratch
    for M, N, K in ((256, 4096, 14336), (32, 4096, 14336), (17, 1000, 14336), (5, 300, 4096)):
        need = tb.tbik_gemm_workspace_bytes(M, N, K)
        say("noalloc", M, N, K, "workspace bytes", need)
        assert need <= cap
        A = inputs.normal_bf16((M, K), 15000 + M, device=DEV)
        W = inputs.normal_bf16((N, K), 15001 + N, std=0.02, device=DEV)
        ref, refb = tb.tbik_gemm(A, W, want_bf16=True)
        got, gotb = tb.tbik_gemm_noalloc(A, W, want_bf16=True)
        assert np.array_equal(_u32(got), _u32(ref)), (M, N, K)
        assert torch.equal(gotb.view(torch.int16), refb.view(torch.int16)), (M, N, K)
    # a shape whose partials exceed the scratch is refused before any launch
    big = (256, 16384, 14336)
    assert tb.tbik_gemm_workspace_bytes(*big) > cap
    A = torch.empty((big[0], big[2]), dtype=torch.bfloat16, device=DEV)
    W = torch.empty((big[1], big[2]), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tb.TbikError) as e:
        tb.tbik_gemm_noalloc(A, W)
    assert e.value.code == -5
