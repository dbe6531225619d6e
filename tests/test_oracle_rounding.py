"""Pins of the oracle's rounding-location variants (rounding-alignment
article, "the problem" and "three nodes").

"once" keeps fp32 intermediates and rounds at the node's bf16 output;
"each_op" is the misaligned stack read as eager bf16 tensor arithmetic.
Both are checked bit for bit against torch's CPU bf16 tensor arithmetic,
which rounds every elementwise operation to bf16 (the library routine the
"each_op" reading names), on inputs where no reduction order can matter;
the fp32 activation comes from the oracle's EXP primitive, which is pinned
elsewhere.  Each test also shows the two variants differ on its inputs, so
the check would see a dropped or misplaced rounding.
"""
import numpy as np
import pytest
import torch

from tp_invariant_numerics_amd import inputs

BF = torch.bfloat16


def _t(bits):
    """uint16 bf16 bit patterns -> torch bf16 tensor (CPU)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(BF)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf_bits(a):
    return _bits(torch.from_numpy(np.asarray(a, np.float32)).to(BF))


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def test_rope_each_op_equals_eager_bf16(orc):
    """Rotate-half RoPE on bf16 tensors with bf16 cos/sin (each product,
    the sum and the difference rounded): q*cos + rotate_half(q)*sin."""
    T, heads, hd = 96, 3, 128
    x = _bits(inputs.normal_bf16((T, heads, hd), 7100))
    pos = (np.arange(T, dtype=np.int32) * 337) % 4096
    c, s = orc.rope_table(1e6, hd, 4096)
    got = orc.rope(x, pos, c, s, rounding="each_op")
    q = _t(x)
    cb = torch.from_numpy(np.concatenate([c[pos], c[pos]], -1)).to(BF)[:, None, :]
    sb = torch.from_numpy(np.concatenate([s[pos], s[pos]], -1)).to(BF)[:, None, :]
    rot = torch.cat([-q[..., hd // 2:], q[..., :hd // 2]], dim=-1)
    ref = q * cb + rot * sb
    assert np.array_equal(got, _bits(ref))
    once = orc.rope(x, pos, c, s)
    assert np.count_nonzero(once != got) > T      # the rounding location matters
    # fp32 reference of the aligned node, rounded once
    qf = q.float()
    ref_once = (qf * torch.from_numpy(np.concatenate([c[pos], c[pos]], -1))[:, None, :]
                + torch.cat([-qf[..., hd // 2:], qf[..., :hd // 2]], -1)
                * torch.from_numpy(np.concatenate([s[pos], s[pos]], -1))[:, None, :])
    assert np.array_equal(once, _bits(ref_once.to(BF)))


def _sparse_norm_inputs(rows, H, seed):
    """Rows with 8 nonzero positions: x integers in [128, 255] (exact in
    bf16), r quarters, so x + r is exact in fp32 but not in bf16, and every
    sum of squares (aligned or not) is an exact fp32 integer or quarter sum
    below 2^24 -- the reduction order cannot change it."""
    rng = np.random.default_rng(seed)
    x = np.zeros((rows, H), np.float32)
    r = np.zeros((rows, H), np.float32)
    for i in range(rows):
        cols = rng.choice(H, 8, replace=False)
        x[i, cols] = rng.integers(128, 256, 8) * rng.choice([-1.0, 1.0], 8)
        r[i, cols] = rng.integers(1, 4, 8) * 0.25
    w = rng.integers(1, 64, H).astype(np.float32) / 32.0        # exact in bf16
    return _bf_bits(x), _bf_bits(r), _bf_bits(w)


@pytest.mark.parametrize("rounding", ["once", "each_op"])
def test_rmsnorm_rounding_equals_eager(orc, rounding):
    rows, H, eps = 24, 4096, 1e-6
    x, r, w = _sparse_norm_inputs(rows, H, 7200)
    y, r_out = orc.rmsnorm_residual(x, r, w, eps, rounding=rounding)
    xt, rt, wt = _t(x), _t(r), _t(w)
    if rounding == "each_op":
        h = (xt + rt).float()                         # bf16 add, then fp32
    else:
        h = xt.float() + rt.float()
    var = (h * h).sum(-1, keepdim=True) / H           # exact: see the input recipe
    rstd = 1.0 / torch.sqrt(var + torch.tensor(eps, dtype=torch.float32))
    n = h * rstd
    if rounding == "each_op":
        ref = wt * n.to(BF)                           # bf16 multiply
    else:
        ref = (n * wt.float()).to(BF)
    assert np.array_equal(y, _bits(ref))
    assert np.array_equal(r_out, _bits(h.to(BF)))


def test_rmsnorm_variants_differ(orc):
    x, r, w = _sparse_norm_inputs(24, 4096, 7200)
    y0, r0 = orc.rmsnorm_residual(x, r, w, 1e-6)
    y1, r1 = orc.rmsnorm_residual(x, r, w, 1e-6, rounding="each_op")
    assert np.array_equal(r0, r1)                     # the residual is bf16 either way
    assert np.count_nonzero(y0 != y1) > 0


def test_swiglu_each_op_equals_eager(orc):
    """bf16(bf16(silu(g)) * u): silu in fp32 from the pinned EXP primitive
    with one IEEE division (numpy binary32), then torch bf16 arithmetic."""
    g = _bits(inputs.normal_bf16((64, 512), 7300, std=3.0))
    u = _bits(inputs.normal_bf16((64, 512), 7301))
    got = orc.swiglu(g, u, rounding="each_op")
    gf = orc.bf16_to_f32(g).astype(np.float32)
    den = np.float32(1.0) + orc.expf(-gf).reshape(gf.shape).astype(np.float32)
    silu = (gf / den).astype(np.float32)
    ref = torch.from_numpy(silu).to(BF) * _t(u)
    assert np.array_equal(got, _bits(ref))
    once = orc.swiglu(g, u)
    assert np.array_equal(once, _bits((torch.from_numpy(silu) * _t(u).float()).to(BF)))
    assert np.count_nonzero(once != got) > 100


def test_swiglu_each_op_special_cases(orc):
    """u = +-2^k: scaling commutes with rounding, so both variants agree."""
    g = _bits(inputs.normal_bf16((8, 256), 7302, std=4.0))
    for ub in (0x3F80, 0x4000, 0xBE80):                    # 1, 2, -0.25
        u = np.full_like(g, ub)
        assert np.array_equal(orc.swiglu(g, u), orc.swiglu(g, u, rounding="each_op"))
