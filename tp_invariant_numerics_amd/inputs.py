"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the method's arithmetic: it only draws random
numbers and lets PyTorch convert them to bfloat16 (round-to-nearest-even).
The same tensor is then handed to both the GPU library and the CPU oracle.

Distributions follow the transformer-shaped workloads the method is
evaluated on: activations ~N(0,1), weights ~N(0,0.02), residual inputs with
1% outliers scaled by 100, RMSNorm weights ~N(1,0.1), uniform integer
targets, positions 0..max_pos-1 (optionally shuffled).
"""
import numpy as np
import torch


def _gen(seed):
    return np.random.Generator(np.random.PCG64(int(seed)))


def _cuda_gen(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, seed, std=1.0, mean=0.0, device="cpu"):
    """bf16 tensor with entries ~N(mean, std^2)."""
    shape = tuple(int(s) for s in shape)
    if str(device).startswith("cuda"):
        x = torch.randn(shape, generator=_cuda_gen(seed), device=device, dtype=torch.float32)
    else:
        x = torch.from_numpy(_gen(seed).standard_normal(shape, dtype=np.float32))
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return x.to(torch.bfloat16)


def outlier_bf16(shape, seed, p=0.01, scale=100.0, device="cpu"):
    """~N(0,1) bf16 with each entry independently multiplied by `scale` with
    probability `p` (independent Bernoulli mask per tensor)."""
    shape = tuple(int(s) for s in shape)
    if str(device).startswith("cuda"):
        g = _cuda_gen(seed)
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    else:
        g = _gen(seed)
        x = torch.from_numpy(g.standard_normal(shape, dtype=np.float32))
        u = torch.from_numpy(g.random(shape, dtype=np.float32))
    x = torch.where(u < p, x * scale, x)
    return x.to(torch.bfloat16)


def uniform_int(n, high, seed, device="cpu"):
    """int32 tensor of n values uniform in [0, high)."""
    if str(device).startswith("cuda"):
        return torch.randint(0, int(high), (int(n),), generator=_cuda_gen(seed), device=device,
                             dtype=torch.int32)
    return torch.from_numpy(_gen(seed).integers(0, int(high), int(n), dtype=np.int32))


def positions(n, max_pos, seed=None):
    """Positions 0..n-1 modulo max_pos, shuffled when a seed is given."""
    p = np.arange(int(n), dtype=np.int64) % int(max_pos)
    if seed is not None:
        p = _gen(seed).permutation(p)
    return torch.from_numpy(p.astype(np.int32))


def integer_bf16(shape, seed, lo=-8, hi=8):
    """bf16 tensor of small integers in [lo, hi] (exactly representable)."""
    shape = tuple(int(s) for s in shape)
    x = _gen(seed).integers(lo, hi + 1, shape).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def one_per_block_bf16(shape, seed, block=64, spread=6, value=None, device="cpu"):
    """bf16 tensor whose rows hold exactly one nonzero entry in each `block`-wide
    slice of the last axis, at a uniform position.  Values ~N(0,1) times
    2^e with e uniform in [-spread, spread], or the constant `value`.  Against
    any dense second operand, every `block`-wide partial dot product of such a
    row has a single nonzero term."""
    shape = tuple(int(s) for s in shape)
    rows, n = int(np.prod(shape[:-1])), shape[-1]
    nblk = (n + block - 1) // block
    g = _gen(seed)
    x = np.zeros((rows, nblk * block), np.float32)
    pos = g.integers(0, block, (rows, nblk)) + np.arange(nblk) * block
    if value is None:
        v = g.standard_normal((rows, nblk)).astype(np.float32)
        v = v * np.exp2(g.integers(-spread, spread + 1, (rows, nblk))).astype(np.float32)
        v[v == 0] = 1.0
    else:
        v = np.full((rows, nblk), value, np.float32)
    np.put_along_axis(x, pos, v, axis=1)
    # a ragged last block keeps its entry only if it falls inside
    t = torch.from_numpy(np.ascontiguousarray(x[:, :n]).reshape(shape)).to(torch.bfloat16)
    return t.to(device)


def bits(t):
    """numpy uint16 view of a bf16 tensor's bit patterns (copied to host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(b):
    """bf16 tensor from numpy uint16 bit patterns."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)


# --- decoder composition -------------------------------------------------------

class DecoderConfig:
    """Shape of the random-init decoder (pre-norm, RMSNorm + RoPE attention,
    SwiGLU MLP, untied LM head)."""

    def __init__(self, layers=8, d=2048, heads=16, head_dim=128, ffn=5632, vocab=32000,
                 theta=1e6, eps=1e-6):
        self.layers, self.d, self.heads, self.head_dim = layers, d, heads, head_dim
        self.ffn, self.vocab, self.theta, self.eps = ffn, vocab, theta, eps
        assert heads * head_dim == d

    def __repr__(self):
        return ("DecoderConfig(layers=%d, d=%d, heads=%d, head_dim=%d, ffn=%d, vocab=%d)"
                % (self.layers, self.d, self.heads, self.head_dim, self.ffn, self.vocab))


def decoder_weights(cfg, seed, device="cpu", std=0.02):
    """bf16 weights ~N(0, std^2) in the nn.Linear [out, in] layout; RMSNorm
    weights are ones.  Per layer: w_qk [2d, d] (query rows then key rows),
    w_v [d, d], w_o [d, d], w_gu [2 ffn, d] (gate rows then up rows),
    w_down [d, ffn]."""
    d, f = cfg.d, cfg.ffn
    ones = torch.ones((d,), dtype=torch.bfloat16, device=device)
    w = {"emb": normal_bf16((cfg.vocab, d), seed, std=std, device=device),
         "lm_head": normal_bf16((cfg.vocab, d), seed + 1, std=std, device=device),
         "final_norm": ones, "layers": []}
    for l in range(cfg.layers):
        s = seed + 16 * (l + 1)
        w["layers"].append({
            "attn_norm": ones, "mlp_norm": ones,
            "w_qk": normal_bf16((2 * d, d), s, std=std, device=device),
            "w_v": normal_bf16((d, d), s + 1, std=std, device=device),
            "w_o": normal_bf16((d, d), s + 2, std=std, device=device),
            "w_gu": normal_bf16((2 * f, d), s + 3, std=std, device=device),
            "w_down": normal_bf16((d, f), s + 4, std=std, device=device),
        })
    return w


def decoder_tokens(batch, length, vocab, seed, device="cpu"):
    """[batch, length] int32 token ids, uniform over the vocabulary."""
    return uniform_int(batch * length, vocab, seed, device=device).view(batch, length)
