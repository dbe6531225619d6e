"""Oracle decoder forward -- TEST INFRASTRUCTURE (tests, smoke check and the
benchmark's CPU leg only).

The plain composition of the oracle's nodes into a pre-norm decoder (TBIK
summary page, "technical framework": the invariant GEMM and reductions
inside a model; rounding-alignment article, "three nodes": fp32
intermediates, one bf16 rounding per node output).  Every GEMM uses the
scalar leaf, so this defines, bit for bit, what the library's decoder
composition in scalar-leaf mode must return.  Written from the definitions,
not from the library's composition:

  layer:  h = RMSNorm(x + resid)          (resid <- bf16(x + resid))
          Q = bf16(h Wq^T), K = bf16(h Wk^T), V = bf16(h Wv^T)
          Q, K rotated (RoPE, rotate-half, positions 0..L-1 per sequence)
          per sequence and head: S = Q K^T (fp32), P = causal softmax of
          S * fp32(1/sqrt(head_dim)) (bf16), O = bf16(P V)
          x = bf16(O Wo^T)                 (K split into tp shards)
          h = RMSNorm(x + resid)
          a = SwiGLU(bf16(h Wg^T), bf16(h Wu^T))
          x = bf16(a Wdown^T)              (K split into tp shards)
  final:  h = RMSNorm(x + resid); logits = h Wlm^T (fp32);
          lp[t] = log-softmax(logits[t])[token[t+1]]  (vocab split in tp)

Weights and tokens are numpy uint16 bf16 bit patterns / int32.
"""
import numpy as np

from . import (gemm, gemm_tpsim, rmsnorm_residual, rope_table, rope, swiglu,
               softmax_causal, logsoftmax_gather, f32_to_bf16)


def _lin(x, w, tp=1):
    """bf16(x w^T); the reduction over K split into tp tree shards."""
    if tp == 1:
        return f32_to_bf16(gemm(x, w))
    return f32_to_bf16(gemm_tpsim(x, w, tp)[0])


NODES = ("rmsnorm", "rope", "swiglu")


def decoder_logprobs(w, tokens, cfg, tp=1, rounding=None):
    """tokens [B, L] int32 -> [B, L-1] fp32 log-probabilities of tokens[:, 1:].

    rounding: optional {node: "once" | "each_op"} for the nodes RMSNorm, RoPE
    and SwiGLU (rounding-alignment article, "three nodes"); default "once"."""
    rd = dict.fromkeys(NODES, "once")
    rd.update(rounding or {})
    tokens = np.asarray(tokens, np.int32)
    B, L = tokens.shape
    d, H, hd, f = cfg.d, cfg.heads, cfg.head_dim, cfg.ffn
    T = B * L
    scale = np.float32(1.0 / np.sqrt(np.float64(hd)))      # fp32 of 1/sqrt(head_dim)
    cos_t, sin_t = rope_table(cfg.theta, hd, L)
    pos = np.tile(np.arange(L, dtype=np.int32), B)

    x = w["emb"][tokens.reshape(-1)]
    resid = np.zeros((T, d), np.uint16)
    for lw in w["layers"]:
        h, resid = rmsnorm_residual(x, resid, lw["attn_norm"], cfg.eps, rd["rmsnorm"])
        wq, wk = lw["w_qk"][:d], lw["w_qk"][d:]
        q = rope(_lin(h, wq).reshape(T, H, hd), pos, cos_t, sin_t, rd["rope"])
        k = rope(_lin(h, wk).reshape(T, H, hd), pos, cos_t, sin_t, rd["rope"])
        v = _lin(h, lw["w_v"]).reshape(T, H, hd)
        o = np.empty((T, H, hd), np.uint16)
        for b in range(B):
            rows = slice(b * L, (b + 1) * L)
            for j in range(H):
                S = gemm(q[rows, j], k[rows, j])                   # [L, L] fp32
                P = softmax_causal(S, 0, scale)                    # [L, L] bf16
                o[rows, j] = f32_to_bf16(gemm(P, v[rows, j].T))    # P V
        x = _lin(o.reshape(T, d), lw["w_o"], tp)
        h, resid = rmsnorm_residual(x, resid, lw["mlp_norm"], cfg.eps, rd["rmsnorm"])
        g = _lin(h, lw["w_gu"][:f])
        u = _lin(h, lw["w_gu"][f:])
        x = _lin(swiglu(g, u, rd["swiglu"]), lw["w_down"], tp)
    h, _ = rmsnorm_residual(x, resid, w["final_norm"], cfg.eps, rd["rmsnorm"])
    logits = gemm(h, w["lm_head"])
    targets = np.zeros((B, L), np.int32)
    targets[:, :L - 1] = tokens[:, 1:]
    lp, _ = logsoftmax_gather(logits, targets.reshape(-1), tp)
    return lp.reshape(B, L)[:, :L - 1]
