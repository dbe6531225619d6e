"""Decoder composition: a pre-norm transformer forward built only from the
library's kernels, returning the log-probabilities of the next tokens.

This is the setting in which the pages measure the method: the logprobs of
a trainer and of an inference engine must agree bit for bit (TBIK summary
page, Abstract and "technical framework"; rounding-alignment article,
"three nodes").  Each layer is

    h, resid = RMSNorm(x + resid)                    tbik_rmsnorm_residual
    q | k    = h W_qk^T,   V^T = W_v h^T             tbik_gemm (bf16 out)
    q, k     = RoPE(q), RoPE(k)                      tbik_rope (in place)
    S        = q k^T per (sequence, head)            tbik_gemm_strided_batched
    P        = causal softmax(S / sqrt(head_dim))    tbik_softmax_causal
    O        = P V per (sequence, head)              tbik_gemm_strided_batched
               (MFMA mode: the three in one kernel,  tbik_attention_causal)
    x        = O W_o^T                               row-parallel: tp K shards
    h, resid = RMSNorm(x + resid)
    g | u    = h W_gu^T;  a = SwiGLU(g, u)           tbik_gemm, tbik_swiglu
    x        = a W_down^T                            row-parallel: tp K shards

then RMSNorm, the LM head (fp32 logits, with the exact row maxima fused into
its epilogue in MFMA mode) and the tree log-softmax with the next-token
gather, its vocabulary split in tp shards.

Simulated tensor parallelism touches exactly the reductions real tensor
parallelism would split: the K dimension of the two row-parallel GEMMs and
the vocabulary of the log-softmax.  Column-parallel GEMMs and attention heads
are independent per rank and need no change.  V is produced already
transposed (its GEMM with the operands swapped), so P V needs no transpose
kernel.  Python only allocates buffers and passes pointers; every step runs
in libtbik.
"""
import math

import torch

from . import lib, _chk, _stream, LEAF_MFMA, ROUNDING
from .inputs import DecoderConfig  # noqa: F401  (re-exported for callers)

__all__ = ["decoder_forward", "DecoderConfig", "NODES"]

# the three nodes whose rounding location the rounding-alignment article
# studies; each is "once" (fp32 intermediates) or "each_op" (eager bf16)
NODES = ("rmsnorm", "rope", "swiglu")


def _rounding_codes(rounding):
    rd = dict.fromkeys(NODES, "once")
    if rounding:
        unknown = set(rounding) - set(NODES)
        if unknown:
            raise ValueError("unknown rounding nodes: %s" % sorted(unknown))
        rd.update(rounding)
    return {k: ROUNDING[v] for k, v in rd.items()}


_ERR_SHAPE = -2          # TBIK_ERR_SHAPE


def _p(t, off=0):
    return t.data_ptr() + off * t.element_size()


def _gemm(A, lda, W, ldw, C, Cb, ldc, M, N, K, leaf, aoff=0, woff=0, coff=0):
    rc = lib().tbik_gemm(_p(A, aoff), lda, _p(W, woff), ldw,
                         None if C is None else _p(C, coff), ldc,
                         None if Cb is None else _p(Cb, coff), M, N, K, leaf, None, 0,
                         _stream())
    _chk(rc, "tbik_gemm")


def _gemm_rowpar(A, W, out_bf16, tp, leaf, ws):
    """Row-parallel projection: K split into tp shards, tree-combined."""
    M, K = A.shape
    N = W.shape[0]
    if tp == 1:
        _gemm(A, A.stride(0), W, W.stride(0), None, out_bf16, out_bf16.stride(0), M, N, K, leaf)
        return
    rc = lib().tbik_gemm_tpsim(_p(A), A.stride(0), _p(W), W.stride(0), None, out_bf16.stride(0),
                               _p(out_bf16), M, N, K, tp, leaf, _p(ws),
                               ws.numel() * ws.element_size(), _stream())
    _chk(rc, "tbik_gemm_tpsim")


_ROPE = {}


def _rope_tables(theta, hd, L, dev):
    """cos/sin tables for positions 0..L-1, built once on the host per shape."""
    key = (theta, hd, L, str(dev))
    if key not in _ROPE:
        c = torch.empty((L, hd // 2), dtype=torch.float32)
        s = torch.empty((L, hd // 2), dtype=torch.float32)
        _chk(lib().tbik_rope_table(theta, hd, L, c.data_ptr(), s.data_ptr()), "tbik_rope_table")
        _ROPE[key] = (c.to(dev), s.to(dev))
    return _ROPE[key]


def decoder_forward(weights, tokens, cfg, tp=1, leaf_mode=LEAF_MFMA, rounding=None,
                    rowpar=None):
    """tokens [B, L] int32 on the device -> logprobs [B, L-1] fp32 of
    tokens[:, 1:] given their prefixes.  rounding: optional {node: "once" |
    "each_op"} for the nodes in NODES (default: all "once").  rowpar:
    optional callable (A, W, out_bf16, tp) replacing the library's
    row-parallel projection, for comparisons against other reduction
    orders; None (the default) uses the tree."""
    rc_of = _rounding_codes(rounding)
    B, L = tokens.shape
    d, H, hd, f, V = cfg.d, cfg.heads, cfg.head_dim, cfg.ffn, cfg.vocab
    T = B * L
    dev = tokens.device
    L_ = lib()
    bf, f32 = torch.bfloat16, torch.float32
    x = torch.empty((T, d), dtype=bf, device=dev)
    resid = torch.zeros((T, d), dtype=bf, device=dev)
    resid2 = torch.empty((T, d), dtype=bf, device=dev)
    h = torch.empty((T, d), dtype=bf, device=dev)
    qk = torch.empty((T, 2 * d), dtype=bf, device=dev)
    vT = torch.empty((d, T), dtype=bf, device=dev)
    S = torch.empty((H, L, L), dtype=f32, device=dev)
    P = torch.empty((H, L, L), dtype=bf, device=dev)
    attn = torch.empty((T, d), dtype=bf, device=dev)
    gu = torch.empty((T, 2 * f), dtype=bf, device=dev)
    a = torch.empty((T, f), dtype=bf, device=dev)
    ws = torch.empty((tp, T, d), dtype=f32, device=dev) if tp > 1 else None
    logits = torch.empty((T, V), dtype=f32, device=dev)
    tok = tokens.reshape(-1).contiguous()
    pos = torch.arange(L, dtype=torch.int32, device=dev).repeat(B)
    c_tab, s_tab = _rope_tables(float(cfg.theta), hd, L, dev)
    scale = float(torch.tensor(1.0 / math.sqrt(hd), dtype=f32))
    st = _stream()

    emb = weights["emb"]
    _chk(L_.tbik_gather_rows(_p(emb), emb.stride(0), V, _p(tok), T, d, _p(x), d, st),
         "tbik_gather_rows")

    def norm(xin, w):
        nonlocal resid, resid2
        rc = L_.tbik_rmsnorm_residual_ex(_p(xin), _p(resid), _p(w), _p(h), _p(resid2), T, d, d,
                                         float(cfg.eps), rc_of["rmsnorm"], st)
        _chk(rc, "tbik_rmsnorm_residual_ex")
        resid, resid2 = resid2, resid

    for lw in weights["layers"]:
        norm(x, lw["attn_norm"])
        _gemm(h, d, lw["w_qk"], d, None, qk, 2 * d, T, 2 * d, d, leaf_mode)
        _gemm(lw["w_v"], d, h, d, None, vT, T, d, T, d, leaf_mode)
        # q and k rotated in place by one call: a qk row is the H query heads
        # followed by the H key heads, so it is 2H heads at the same position
        rc = L_.tbik_rope_ex(_p(qk), _p(qk), _p(pos), _p(c_tab), _p(s_tab), T, 2 * H, hd, 2 * d,
                             L, rc_of["rope"], st)
        _chk(rc, "tbik_rope_ex")
        if leaf_mode == LEAF_MFMA and hd == 128 and L in (64, 128, 256, 512):
            # fused kernel: the same bits as the three steps below, without
            # the score matrix in HBM
            rc = L_.tbik_attention_causal(_p(qk), 2 * d, _p(qk, d), 2 * d, _p(vT), T, _p(attn), d,
                                          L, H, hd, B, scale, st)
            _chk(rc, "tbik_attention_causal")
        else:
            for b in range(B):
                r0 = b * L
                rc = L_.tbik_gemm_strided_batched(
                    _p(qk, r0 * 2 * d), 2 * d, hd, _p(qk, r0 * 2 * d + d), 2 * d, hd,
                    _p(S), L, L * L, None, L, L, hd, H, leaf_mode, st)
                _chk(rc, "tbik_gemm_strided_batched")
                rc = L_.tbik_softmax_causal(_p(S), L, L * L, _p(P), L, L * L, L, L, H, 0, scale,
                                            st)
                _chk(rc, "tbik_softmax_causal")
                rc = L_.tbik_gemm_strided_batched(
                    _p(P), L, L * L, _p(vT, r0), T, hd * T,
                    None, d, hd, _p(attn, r0 * d), L, hd, L, H, leaf_mode, st)
                _chk(rc, "tbik_gemm_strided_batched")
        if rowpar is None:
            _gemm_rowpar(attn, lw["w_o"], x, tp, leaf_mode, ws)
        else:
            rowpar(attn, lw["w_o"], x, tp)
        norm(x, lw["mlp_norm"])
        # gate/up projection and SwiGLU: one fused launch where the library
        # takes the shape (same bits as the two calls below)
        rc = (L_.tbik_gemm_swiglu(_p(h), d, _p(lw["w_gu"]), d, _p(a), f, T, f, d,
                                  rc_of["swiglu"], st)
              if leaf_mode == LEAF_MFMA else _ERR_SHAPE)
        if rc == _ERR_SHAPE:
            _gemm(h, d, lw["w_gu"], d, None, gu, 2 * f, T, 2 * f, d, leaf_mode)
            rc = L_.tbik_swiglu_ex(_p(gu), _p(gu, f), _p(a), T, f, 2 * f, 2 * f, f,
                                   rc_of["swiglu"], st)
        _chk(rc, "tbik_gemm_swiglu / tbik_swiglu_ex")
        if rowpar is None:
            _gemm_rowpar(a, lw["w_down"], x, tp, leaf_mode, ws)
        else:
            rowpar(a, lw["w_down"], x, tp)
    norm(x, weights["final_norm"])
    lm = weights["lm_head"]
    targets = torch.zeros((B, L), dtype=torch.int32, device=dev)
    targets[:, :L - 1] = tokens[:, 1:]
    targets = targets.reshape(-1)
    lp = torch.empty((T,), dtype=f32, device=dev)
    lws = torch.empty((T * tp,), dtype=f32, device=dev)
    if leaf_mode == LEAF_MFMA:
        # row maxima fused into the LM-head GEMM: the log-softmax reads the
        # logits once
        nblk = (V + 63) // 64
        pmax = torch.empty((T, nblk), dtype=f32, device=dev)
        _chk(L_.tbik_gemm_logits(_p(h), d, _p(lm), lm.stride(0), _p(logits), V, T, V, d,
                                 _p(pmax), nblk, st), "tbik_gemm_logits")
        rc = L_.tbik_logsoftmax_gather_pmax(_p(logits), V, _p(targets), _p(lp), T, V, tp,
                                            _p(pmax), nblk, nblk, _p(lws), lws.numel() * 4, st)
        _chk(rc, "tbik_logsoftmax_gather_pmax")
    else:
        _gemm(h, d, lm, lm.stride(0), logits, None, V, T, V, d, leaf_mode)
        rc = L_.tbik_logsoftmax_gather(_p(logits), V, _p(targets), _p(lp), T, V, tp, _p(lws),
                                       lws.numel() * 4, st)
        _chk(rc, "tbik_logsoftmax_gather")
    return lp.view(B, L)[:, :L - 1]
