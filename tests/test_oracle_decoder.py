"""Pins of the oracle's decoder composition (CPU).

The composition is pinned by (1) a plain binary64 decoder written here from
the same layer definition, which must agree to bf16 rounding noise, with
planted wiring mistakes (no causal mask, no RoPE, interleaved instead of
rotate-half pairs) shown to exceed that tolerance by a wide margin;
(2) causality; (3) batch invariance; (4) tp invariance (TBIK summary page,
Abstract: identical results whatever the TP size and batch).

Tolerance: each node output is rounded to bf16 (relative error <= 2^-9);
a 2-layer forward has about 25 such nodes between the embedding and the
logits, and the logits of this configuration are O(1..10), so logprob
differences of a few 1e-2 are rounding noise.  The planted mistakes move
logprobs by O(1).
"""
import numpy as np
import pytest

from tp_invariant_numerics_amd import inputs
from oracle import decoder as od

CFG = inputs.DecoderConfig(layers=2, d=256, heads=2, head_dim=128, ffn=512, vocab=1000)
MEAN_TOL, MAX_TOL = 0.05, 0.25


def _np_weights(w):
    b = inputs.bits
    return {"emb": b(w["emb"]), "lm_head": b(w["lm_head"]), "final_norm": b(w["final_norm"]),
            "layers": [{k: b(v) for k, v in lw.items()} for lw in w["layers"]]}


@pytest.fixture(scope="module")
def setup():
    w = _np_weights(inputs.decoder_weights(CFG, 777, std=0.1))
    tok = inputs.decoder_tokens(2, 64, CFG.vocab, 778).numpy()
    return w, tok, od.decoder_logprobs(w, tok, CFG)


def f64_decoder(w, tokens, cfg, mask=True, use_rope=True, interleave=False):
    """Unrounded binary64 forward of the same layer definition."""
    F = lambda a: (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)
    B, L = tokens.shape
    d, H, hd, ff = cfg.d, cfg.heads, cfg.head_dim, cfg.ffn
    T = B * L
    half = hd // 2
    inv = cfg.theta ** (-np.arange(half) * 2.0 / hd)
    ang = np.tile(np.arange(L), B)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]

    def norm(hs, wn):
        return hs / np.sqrt(np.mean(hs * hs, axis=1, keepdims=True) + cfg.eps) * F(wn)

    def rope(q):
        if not use_rope:
            return q
        if interleave:
            a, b = q[..., 0::2], q[..., 1::2]
            out = np.empty_like(q)
            out[..., 0::2] = a * c - b * s
            out[..., 1::2] = b * c + a * s
            return out
        a, b = q[..., :half], q[..., half:]
        return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)

    x = F(w["emb"])[tokens.reshape(-1)]
    resid = np.zeros((T, d))
    for lw in w["layers"]:
        resid = x + resid
        h = norm(resid, lw["attn_norm"])
        wqk = F(lw["w_qk"])
        q = rope((h @ wqk[:d].T).reshape(T, H, hd))
        k = rope((h @ wqk[d:].T).reshape(T, H, hd))
        v = (h @ F(lw["w_v"]).T).reshape(T, H, hd)
        o = np.empty((T, H, hd))
        for b in range(B):
            r = slice(b * L, (b + 1) * L)
            for j in range(H):
                S = q[r, j] @ k[r, j].T / np.sqrt(hd)
                if mask:
                    S = np.where(np.tril(np.ones((L, L))) > 0, S, -np.inf)
                S = S - S.max(axis=1, keepdims=True)
                P = np.exp(S)
                o[r, j] = (P / P.sum(axis=1, keepdims=True)) @ v[r, j]
        x = o.reshape(T, d) @ F(lw["w_o"]).T
        resid = x + resid
        h = norm(resid, lw["mlp_norm"])
        wgu = F(lw["w_gu"])
        g, u = h @ wgu[:ff].T, h @ wgu[ff:].T
        x = (g / (1 + np.exp(-g)) * u) @ F(lw["w_down"]).T
    resid = x + resid
    lg = norm(resid, w["final_norm"]) @ F(w["lm_head"]).T
    m = lg.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(lg - m).sum(axis=1))
    tgt = np.concatenate([tokens[:, 1:], np.zeros((B, 1), np.int32)], axis=1).reshape(-1)
    return (lg[np.arange(T), tgt] - lse).reshape(B, L)[:, :L - 1]


def test_decoder_matches_binary64(setup):
    w, tok, lp = setup
    err = np.abs(lp.astype(np.float64) - f64_decoder(w, tok, CFG))
    assert err.mean() <= MEAN_TOL and err.max() <= MAX_TOL, (err.mean(), err.max())


@pytest.mark.parametrize("mistake", [dict(mask=False), dict(use_rope=False),
                                     dict(interleave=True)])
def test_planted_wiring_mistakes_are_detected(setup, mistake):
    w, tok, lp = setup
    err = np.abs(lp.astype(np.float64) - f64_decoder(w, tok, CFG, **mistake))
    assert err.mean() > 10 * MEAN_TOL


def test_decoder_causal(setup):
    w, tok, lp = setup
    j = 40
    tok2 = tok.copy()
    tok2[:, j] = (tok2[:, j] + 1) % CFG.vocab
    lp2 = od.decoder_logprobs(w, tok2, CFG)
    assert np.array_equal(lp[:, :j - 1].view(np.uint32), lp2[:, :j - 1].view(np.uint32))
    assert not np.array_equal(lp[:, j - 1:].view(np.uint32), lp2[:, j - 1:].view(np.uint32))


def test_decoder_batch_invariant(setup):
    w, tok, lp = setup
    lp1 = od.decoder_logprobs(w, tok[1:2], CFG)
    assert np.array_equal(lp[1:2].view(np.uint32), lp1.view(np.uint32))


@pytest.mark.parametrize("tp", [2, 4])
def test_decoder_tp_invariant(setup, tp):
    w, tok, lp = setup
    lpt = od.decoder_logprobs(w, tok, CFG, tp=tp)
    assert np.array_equal(lp.view(np.uint32), lpt.view(np.uint32))


# --------------------------------------------------------------------------
# rounding locations (rounding-alignment article, "three nodes")
# --------------------------------------------------------------------------
@pytest.mark.parametrize("nodes", [("rope",), ("swiglu",), ("rmsnorm",),
                                   ("rmsnorm", "rope", "swiglu")])
def test_decoder_rounding_location_gap(setup, nodes):
    """Rounding the intermediates of a node to bf16 moves the logprobs (the
    train/inference mismatch the article traces to these nodes) but not past
    bf16 rounding noise, and the tree kernels keep every variant tp-invariant."""
    w, tok, lp = setup
    rd = dict.fromkeys(nodes, "each_op")
    lpv = od.decoder_logprobs(w, tok, CFG, rounding=rd)
    assert np.count_nonzero(lpv.view(np.uint32) != lp.view(np.uint32)) > 0
    err = np.abs(lpv.astype(np.float64) - f64_decoder(w, tok, CFG))
    assert err.mean() <= MEAN_TOL and err.max() <= MAX_TOL, (err.mean(), err.max())
    lpt = od.decoder_logprobs(w, tok, CFG, tp=2, rounding=rd)
    assert np.array_equal(lpv.view(np.uint32), lpt.view(np.uint32))


def test_decoder_rounding_once_is_default(setup):
    w, tok, lp = setup
    lpo = od.decoder_logprobs(w, tok, CFG, rounding=dict.fromkeys(od.NODES, "once"))
    assert np.array_equal(lpo.view(np.uint32), lp.view(np.uint32))
