"""The ceiling microbenchmarks compute what they claim to move.

Each kernel's result is checked against the same reduction done on the host,
so a rate quoted from it is the rate of the stated traffic (a kernel whose
loads were dropped or misdirected would fail here):

* tbik_bench_copy_lds: each thread's 16 bytes of the last stage in its
  workgroup's LDS ring, folded by xor, equal the bytes at that place of the
  window (the stage index wraps from 7 * workgroup);
* tbik_bench_hbm_read: each thread's xor over the 16-byte units it streamed;
* tbik_bench_hbm_copy: dst equals src;
* tbik_bench_mfma: finite, and the same bits on a second launch.
"""
import numpy as np
import pytest
import torch

import tp_invariant_numerics_amd as tb

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    tb.lib()


def _rand_bytes(n, seed):
    g = np.random.default_rng(seed)
    return g.integers(0, 1 << 32, size=n // 4, dtype=np.uint64).astype(np.uint32)


@pytest.mark.parametrize("window,stages,blocks", [(1 << 20, 5, 3), (32768, 1, 2), (65536, 7, 9)])
def test_copy_lds_moves_the_window(window, stages, blocks):
    host = _rand_bytes(2 << 20, 7)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    out, moved = tb.tbik_bench_copy_lds(buf, window, stages, blocks)
    torch.cuda.synchronize()
    assert moved == blocks * stages * 32768
    got = out.cpu().numpy().view(np.uint32).reshape(blocks, 512)
    nst = window // 32768
    words = host.reshape(-1, 4)                       # 16-byte units
    for b in range(blocks):
        st = (7 * b + stages - 1) % nst
        unit = words[st * 2048: st * 2048 + 512]
        exp = unit[:, 0] ^ unit[:, 1] ^ unit[:, 2] ^ unit[:, 3]
        assert np.array_equal(got[b], exp), b


@pytest.mark.parametrize("nbytes,blocks", [(1 << 20, 7), ((1 << 20) + 4096 + 48, 3), (4096, 5)])
def test_hbm_read_folds_every_unit(nbytes, blocks):
    host = _rand_bytes(nbytes, 8)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = tb.tbik_bench_hbm_read(buf, blocks)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).reshape(blocks, 256)
    units = host.reshape(-1, 4)
    folded = units[:, 0] ^ units[:, 1] ^ units[:, 2] ^ units[:, 3]
    idx = np.arange(units.shape[0])
    exp = np.zeros((blocks, 256), np.uint32)
    np.bitwise_xor.at(exp, ((idx // 2048) % blocks, idx % 256), folded)
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("nbytes,blocks", [(1 << 20, 5), ((1 << 16) + 16, 3)])
def test_hbm_copy_copies(nbytes, blocks):
    host = _rand_bytes(nbytes, 9)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    dst = torch.zeros_like(src)
    tb.tbik_bench_hbm_copy(src, dst, blocks)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_mfma_loop_is_finite_and_repeatable():
    seed = torch.from_numpy(np.random.default_rng(10).standard_normal(1024).astype(np.float32)
                            ).to(torch.bfloat16).to(DEV)
    out1, fl = tb.tbik_bench_mfma(seed, 4, 16)
    out2, _ = tb.tbik_bench_mfma(seed, 4, 16)
    torch.cuda.synchronize()
    assert fl == 4 * 8 * 8 * 16 * 16384
    assert torch.isfinite(out1).all()
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32))
