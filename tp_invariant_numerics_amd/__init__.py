"""tp_invariant_numerics_amd -- tree-based invariant kernels (TBIK) on MI355X.

Thin Python binding of libtbik.so (C ABI in include/tbik.h).  Every function
here only checks tensor dtypes/devices, allocates outputs with PyTorch and
passes raw device pointers plus the current HIP stream to the library; all
arithmetic runs in the library's HIP kernels.  There is no fallback: if the
library is missing or no GPU is present, the call raises.

Function names mirror the C entry points (``tbik_gemm`` -> ``tbik_gemm``).
"""
import ctypes as C
import os

import torch

from . import build as _build

__all__ = [
    "TbikError", "lib", "tbik_version", "tbik_strerror", "tbik_tree_groups", "tbik_gemm",
    "tbik_gemm_strided_batched", "tbik_gemm_tpsim", "tbik_gemm_tpsim_workspace_bytes",
    "tbik_tree_combine", "tbik_gemm_tp_partials", "tbik_gemm_shard", "tbik_rmsnorm_residual", "tbik_rope", "tbik_rope_table",
    "tbik_swiglu", "tbik_logsoftmax_gather", "tbik_logsoftmax_workspace_bytes",
    "tbik_softmax_causal", "tbik_primitive", "LEAF_MFMA", "LEAF_SCALAR", "ROUNDING",
    "tbik_transpose_bf16", "tbik_gemm_dgrad", "tbik_gemm_wgrad", "tbik_rope_backward",
    "tbik_swiglu_backward", "tbik_rmsnorm_backward",
]

LEAF_MFMA = 0
LEAF_SCALAR = 1
PRIM_EXP, PRIM_LOG, PRIM_BF16, PRIM_SILU = 0, 1, 2, 3
# rounding location of RMSNorm, RoPE and SwiGLU: fp32 intermediates rounded
# once at the output, or bf16 after every elementwise operation
ROUNDING = {"once": 0, "each_op": 1}

_lib = None


class TbikError(RuntimeError):
    def __init__(self, code, what):
        super().__init__("%s: %s (code %d)" % (what, _strerror(code), code))
        self.code = code


def _strerror(code):
    try:
        return lib().tbik_strerror(code).decode()
    except Exception:  # pragma: no cover - library not loadable
        return "error"


_SIGS = None


def _sigs():
    p, i32, i64, f32, f64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_double, C.c_size_t
    return {
        "tbik_version": (i32, []),
        "tbik_strerror": (C.c_char_p, [i32]),
        "tbik_tree_groups": (i32, [i64]),
        "tbik_gemm_workspace_bytes": (sz, [i32, i32, i32]),
        "tbik_gemm": (i32, [p, i64, p, i64, p, i64, p, i32, i32, i32, i32, p, sz, p]),
        "tbik_gemm_strided_batched": (i32, [p, i64, i64, p, i64, i64, p, i64, i64, p, i32, i32,
                                            i32, i32, i32, p]),
        "tbik_gemm_tpsim_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "tbik_gemm_tpsim": (i32, [p, i64, p, i64, p, i64, p, i32, i32, i32, i32, i32, p, sz, p]),
        "tbik_tree_combine": (i32, [p, i32, p, i64, p, i32, i32, p]),
        "tbik_gemm_tp_partials": (i32, [p, i64, p, i64, p, sz, i32, i32, i32, i32, i32, p]),
        "tbik_gemm_shard": (i32, [p, i64, p, i64, p, i64, i32, i32, i32, i32, i32, p]),
        "tbik_rmsnorm_residual": (i32, [p, p, p, p, p, i32, i32, i64, f32, p]),
        "tbik_rope": (i32, [p, p, p, p, p, i32, i32, i32, i64, i32, p]),
        "tbik_rope_table": (i32, [f64, i32, i32, p, p]),
        "tbik_swiglu": (i32, [p, p, p, i32, i32, i64, i64, i64, p]),
        "tbik_rmsnorm_residual_ex": (i32, [p, p, p, p, p, i32, i32, i64, f32, i32, p]),
        "tbik_rope_ex": (i32, [p, p, p, p, p, i32, i32, i32, i64, i32, i32, p]),
        "tbik_swiglu_ex": (i32, [p, p, p, i32, i32, i64, i64, i64, i32, p]),
        "tbik_gemm_swiglu": (i32, [p, i64, p, i64, p, i64, i32, i32, i32, i32, p]),
        "tbik_logsoftmax_workspace_bytes": (sz, [i32, i32, i32]),
        "tbik_logsoftmax_gather": (i32, [p, i64, p, p, i32, i32, i32, p, sz, p]),
        "tbik_softmax_causal": (i32, [p, i64, i64, p, i64, i64, i32, i32, i32, i32, f32, p]),
        "tbik_primitive": (i32, [i32, p, p, i64, p]),
        "tbik_gemm_logits": (i32, [p, i64, p, i64, p, i64, i32, i32, i32, p, i64, p]),
        "tbik_logsoftmax_gather_pmax": (i32, [p, i64, p, p, i32, i32, i32, p, i64, i32, p, sz,
                                              p]),
        "tbik_gather_rows": (i32, [p, i64, i32, p, i32, i32, p, i64, p]),
        "tbik_attention_causal": (i32, [p, i64, p, i64, p, i64, p, i64, i32, i32, i32, i32, f32,
                                        p]),
        "tbik_transpose_bf16": (i32, [p, i64, p, i64, i32, i32, p]),
        "tbik_gemm_dgrad_workspace_bytes": (sz, [i32, i32, i32]),
        "tbik_gemm_dgrad": (i32, [p, i64, p, i64, p, i64, p, i32, i32, i32, i32, p, sz, p]),
        "tbik_gemm_wgrad_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "tbik_gemm_wgrad": (i32, [p, i64, p, i64, p, i64, i32, i32, i32, i32, i32, p, sz, p]),
        "tbik_rope_backward": (i32, [p, p, p, p, p, i32, i32, i32, i64, i32, p]),
        "tbik_swiglu_backward": (i32, [p, p, p, p, p, i32, i32, i64, i64, i64, i64, i64, p]),
        "tbik_rmsnorm_backward_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "tbik_rmsnorm_backward": (i32, [p, p, p, p, p, p, p, i32, i32, i64, f32, i32, p, sz, p]),
        "tbik_gemm_noalloc_max_bytes": (sz, []),
        "tbik_gemm_noalloc": (i32, [p, i64, p, i64, p, i64, p, i32, i32, i32, i32, p]),
        "tbik_bench_mfma_flops": (i64, [i32, i32]),
        "tbik_bench_mfma": (i32, [p, p, i32, i32, p]),
        "tbik_bench_hbm_read": (i32, [p, i64, p, i32, p]),
        "tbik_bench_hbm_copy": (i32, [p, p, i64, i32, p]),
        "tbik_bench_copy_lds": (i32, [p, i64, i32, p, i32, p]),
    }


def lib():
    """Load libtbik.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError("libtbik.so is not built (%s); run __graft_entry__.build()"
                               % _build.LIB)
        L = C.CDLL(_build.LIB)
        for name, (res, args) in _sigs().items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensor must be on a HIP device")


def _chk(rc, what):
    if rc != 0:
        raise TbikError(rc, what)


def _ld(t):
    """Row stride (elements) of a 2-D tensor with unit column stride."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with contiguous rows")
    return t.stride(0)


def _rows_like(t):
    """An output with t's shape, dtype and leading (row / token) stride: the
    C ABI takes one row stride for an input and the output beside it."""
    rows, ld = t.shape[0], t.stride(0)
    inner = tuple(t.shape[1:])
    n = 1
    for v in inner:
        n *= v
    buf = torch.empty((rows, max(ld, n)), dtype=t.dtype, device=t.device)[:, :n]
    return buf.unflatten(1, inner) if len(inner) > 1 else buf


def _same_rows(out, t, what):
    if out.shape != t.shape or out.stride() != t.stride():
        raise ValueError("%s must have the shape and strides of its input" % what)


def _bits(t):
    if t.dtype != torch.bfloat16:
        raise ValueError("expected bfloat16")
    return t


# --- info -------------------------------------------------------------------

def tbik_version():
    return lib().tbik_version()


def tbik_strerror(code):
    return _strerror(code)


def tbik_tree_groups(n):
    return lib().tbik_tree_groups(n)


# --- GEMM ---------------------------------------------------------------------

def tbik_gemm_workspace_bytes(M, N, K):
    return lib().tbik_gemm_workspace_bytes(M, N, K)


def tbik_gemm(A, W, leaf_mode=LEAF_MFMA, out=None, out_bf16=None, want_fp32=True,
              want_bf16=False, ws="auto"):
    """C = A @ W^T with the tree over 64-wide K blocks.  A [M,K], W [N,K] bf16.
    ws: "auto" allocates the split-K workspace the library asks for, None
    passes none, or a float32 device tensor.
    Returns (C fp32 or None, C_bf16 or None)."""
    _bits(A); _bits(W); _need_gpu(A, W)
    M, K = A.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("K mismatch")
    if out is None and want_fp32:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if out_bf16 is None and want_bf16:
        out_bf16 = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    ref = out if out is not None else out_bf16
    ldc = _ld(ref) if ref is not None else N
    if out is not None and out_bf16 is not None and _ld(out_bf16) != ldc:
        raise ValueError("C and C_bf16 must share the row stride")
    if isinstance(ws, str):
        nb = tbik_gemm_workspace_bytes(M, N, K) if leaf_mode == LEAF_MFMA else 0
        ws = torch.empty((nb // 4,), dtype=torch.float32, device=A.device) if nb else None
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib().tbik_gemm(_ptr(A), _ld(A), _ptr(W), _ld(W), _ptr(out), ldc, _ptr(out_bf16),
                         M, N, K, leaf_mode, _ptr(ws), wsb, _stream())
    _chk(rc, "tbik_gemm")
    return out, out_bf16


def tbik_gemm_noalloc(A, W, leaf_mode=LEAF_MFMA, out=None, out_bf16=None, want_fp32=True,
                      want_bf16=False):
    """tbik_gemm with the split-K partials in the library's own device
    scratch (no workspace argument, nothing allocated by the library)."""
    _bits(A); _bits(W); _need_gpu(A, W)
    M, K = A.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("K mismatch")
    if out is None and want_fp32:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if out_bf16 is None and want_bf16:
        out_bf16 = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    ref = out if out is not None else out_bf16
    ldc = _ld(ref) if ref is not None else N
    if out is not None and out_bf16 is not None and _ld(out_bf16) != ldc:
        raise ValueError("C and C_bf16 must share the row stride")
    rc = lib().tbik_gemm_noalloc(_ptr(A), _ld(A), _ptr(W), _ld(W), _ptr(out), ldc, _ptr(out_bf16),
                                 M, N, K, leaf_mode, _stream())
    _chk(rc, "tbik_gemm_noalloc")
    return out, out_bf16


def tbik_gemm_strided_batched(A, W, leaf_mode=LEAF_MFMA, want_fp32=True, want_bf16=False):
    """A [B,M,K], W [B,N,K] bf16 (contiguous rows) -> (C [B,M,N] fp32, C_bf16)."""
    _bits(A); _bits(W); _need_gpu(A, W)
    B, M, K = A.shape
    N = W.shape[1]
    if A.stride(2) != 1 or W.stride(2) != 1:
        raise ValueError("rows must be contiguous")
    out = torch.empty((B, M, N), dtype=torch.float32, device=A.device) if want_fp32 else None
    outb = torch.empty((B, M, N), dtype=torch.bfloat16, device=A.device) if want_bf16 else None
    rc = lib().tbik_gemm_strided_batched(_ptr(A), A.stride(1), A.stride(0), _ptr(W), W.stride(1),
                                         W.stride(0), _ptr(out), N, M * N, _ptr(outb), M, N, K, B,
                                         leaf_mode, _stream())
    _chk(rc, "tbik_gemm_strided_batched")
    return out, outb


def tbik_gemm_tpsim_workspace_bytes(M, N, K, tp):
    return lib().tbik_gemm_tpsim_workspace_bytes(M, N, K, tp)


def tbik_gemm_tpsim(A, W, tp, leaf_mode=LEAF_MFMA, ws=None, out=None, out_bf16=None,
                    want_bf16=False):
    """Simulated K-sharded GEMM.  Returns (C fp32, C_bf16 or None, ws [tp,M,N])."""
    _bits(A); _bits(W); _need_gpu(A, W)
    M, K = A.shape
    N = W.shape[0]
    if ws is None:
        ws = torch.empty((tp, M, N), dtype=torch.float32, device=A.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if out_bf16 is None and want_bf16:
        out_bf16 = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    rc = lib().tbik_gemm_tpsim(_ptr(A), _ld(A), _ptr(W), _ld(W), _ptr(out), _ld(out),
                               _ptr(out_bf16), M, N, K, tp, leaf_mode, _ptr(ws),
                               ws.numel() * ws.element_size(), _stream())
    _chk(rc, "tbik_gemm_tpsim")
    return out, out_bf16, ws


def tbik_gemm_tp_partials(A, W, tp, leaf_mode=LEAF_MFMA, ws=None):
    """All tp shard partials of the simulated K split -> ws [tp, M, N] fp32."""
    _bits(A); _bits(W); _need_gpu(A, W)
    M, K = A.shape
    N = W.shape[0]
    if ws is None:
        ws = torch.empty((tp, M, N), dtype=torch.float32, device=A.device)
    rc = lib().tbik_gemm_tp_partials(_ptr(A), _ld(A), _ptr(W), _ld(W), _ptr(ws),
                                     ws.numel() * ws.element_size(), M, N, K, tp, leaf_mode,
                                     _stream())
    _chk(rc, "tbik_gemm_tp_partials")
    return ws


def tbik_gemm_shard(A_t, W_t, K_total, tp, leaf_mode=LEAF_MFMA, out=None):
    """One rank's shard node from its own K slice: A_t [M, K_total/tp], W_t [N, K_total/tp]."""
    _bits(A_t); _bits(W_t); _need_gpu(A_t, W_t)
    M = A_t.shape[0]
    N = W_t.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A_t.device)
    rc = lib().tbik_gemm_shard(_ptr(A_t), _ld(A_t), _ptr(W_t), _ld(W_t), _ptr(out), _ld(out), M,
                               N, K_total, tp, leaf_mode, _stream())
    _chk(rc, "tbik_gemm_shard")
    return out


def tbik_tree_combine(ws, out=None, out_bf16=None):
    """ws [tp,M,N] fp32 partials -> top tree -> C [M,N]."""
    _need_gpu(ws)
    tp, M, N = ws.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=ws.device)
    rc = lib().tbik_tree_combine(_ptr(ws), tp, _ptr(out), _ld(out), _ptr(out_bf16), M, N,
                                 _stream())
    _chk(rc, "tbik_tree_combine")
    return out


# --- row ops ------------------------------------------------------------------

def tbik_rmsnorm_residual(x, r, w, eps=1e-6, y=None, r_out=None, want_r_out=True,
                          rounding="once"):
    _bits(x); _bits(r); _bits(w); _need_gpu(x, r, w)
    rows, H = x.shape
    ld = _ld(x)
    if _ld(r) != ld:
        raise ValueError("x and r must share the row stride")
    y = _rows_like(x) if y is None else y
    _same_rows(y, x, "y")
    if r_out is None and want_r_out:
        r_out = _rows_like(x)
    if r_out is not None:
        _same_rows(r_out, x, "r_out")
    rc = lib().tbik_rmsnorm_residual_ex(_ptr(x), _ptr(r), _ptr(w), _ptr(y), _ptr(r_out), rows, H,
                                        ld, float(eps), ROUNDING[rounding], _stream())
    _chk(rc, "tbik_rmsnorm_residual")
    return y, r_out


def tbik_rope(x, pos, cos_tab, sin_tab, y=None, rounding="once"):
    """x [T, heads, d] bf16 (heads contiguous); pos [T] int32; tables [max_pos, d/2]."""
    _bits(x); _need_gpu(x, pos, cos_tab, sin_tab)
    T, heads, d = x.shape
    if x.stride(2) != 1 or x.stride(1) != d:
        raise ValueError("heads must be contiguous with stride head_dim")
    y = _rows_like(x) if y is None else y
    _same_rows(y, x, "y")
    rc = lib().tbik_rope_ex(_ptr(x), _ptr(y), _ptr(pos), _ptr(cos_tab), _ptr(sin_tab), T, heads,
                            d, x.stride(0), cos_tab.shape[0], ROUNDING[rounding], _stream())
    _chk(rc, "tbik_rope")
    return y


def tbik_rope_table(theta, head_dim, max_pos):
    """Host helper: (cos, sin) CPU float32 tensors [max_pos, head_dim/2]."""
    half = head_dim // 2
    c = torch.empty((max_pos, half), dtype=torch.float32)
    s = torch.empty((max_pos, half), dtype=torch.float32)
    rc = lib().tbik_rope_table(float(theta), head_dim, max_pos, _ptr(c), _ptr(s))
    _chk(rc, "tbik_rope_table")
    return c, s


def tbik_gemm_swiglu(A, W_gu, out=None, rounding="once"):
    """H = SwiGLU(bf16(A W_g^T), bf16(A W_u^T)) with W_gu = [W_g; W_u] [2F, K]:
    the gate/up GEMM with the SwiGLU node in its epilogue.  Raises TbikError
    (TBIK_ERR_SHAPE) for shapes the fused kernel does not take."""
    _bits(A); _bits(W_gu); _need_gpu(A, W_gu)
    M, K = A.shape
    F = W_gu.shape[0] // 2
    if W_gu.shape[1] != K or W_gu.shape[0] != 2 * F:
        raise ValueError("W_gu must be [2F, K]")
    if out is None:
        out = torch.empty((M, F), dtype=torch.bfloat16, device=A.device)
    rc = lib().tbik_gemm_swiglu(_ptr(A), _ld(A), _ptr(W_gu), _ld(W_gu), _ptr(out), _ld(out),
                                M, F, K, ROUNDING[rounding], _stream())
    _chk(rc, "tbik_gemm_swiglu")
    return out


def tbik_swiglu(gate, up, out=None, rounding="once"):
    _bits(gate); _bits(up); _need_gpu(gate, up)
    rows, cols = gate.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=gate.device)
    rc = lib().tbik_swiglu_ex(_ptr(gate), _ptr(up), _ptr(out), rows, cols, _ld(gate), _ld(up),
                              _ld(out), ROUNDING[rounding], _stream())
    _chk(rc, "tbik_swiglu")
    return out


def tbik_logsoftmax_workspace_bytes(M, V, tp):
    return lib().tbik_logsoftmax_workspace_bytes(M, V, tp)


def tbik_logsoftmax_gather(logits, targets, tp=1, ws=None, out=None):
    """logits [M,V] fp32, targets [M] int32 -> (lp [M] fp32, ws)."""
    _need_gpu(logits, targets)
    M, V = logits.shape
    nbytes = tbik_logsoftmax_workspace_bytes(M, V, tp)
    if ws is None:
        ws = torch.empty((max(1, nbytes // 4),), dtype=torch.float32, device=logits.device)
    if out is None:
        out = torch.empty((M,), dtype=torch.float32, device=logits.device)
    rc = lib().tbik_logsoftmax_gather(_ptr(logits), _ld(logits), _ptr(targets), _ptr(out), M, V,
                                      tp, _ptr(ws), ws.numel() * 4, _stream())
    _chk(rc, "tbik_logsoftmax_gather")
    return out, ws


def tbik_gemm_logits(A, W, out=None, pmax=None):
    """LM-head GEMM (MFMA leaves) with the row maxima of 64-column blocks
    fused into its epilogue -> (logits [M,N] fp32, pmax [M, ceil(N/64)])."""
    _bits(A); _bits(W); _need_gpu(A, W)
    M, K = A.shape
    N = W.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    nb = (N + 63) // 64
    if pmax is None:
        pmax = torch.empty((M, nb), dtype=torch.float32, device=A.device)
    rc = lib().tbik_gemm_logits(_ptr(A), _ld(A), _ptr(W), _ld(W), _ptr(out), _ld(out), M, N, K,
                                _ptr(pmax), _ld(pmax), _stream())
    _chk(rc, "tbik_gemm_logits")
    return out, pmax


def tbik_logsoftmax_gather_pmax(logits, targets, pmax, tp=1, ws=None, out=None):
    """tbik_logsoftmax_gather taking the row maxima from pmax [M, nb]."""
    _need_gpu(logits, targets, pmax)
    M, V = logits.shape
    nbytes = tbik_logsoftmax_workspace_bytes(M, V, tp)
    if ws is None:
        ws = torch.empty((max(1, nbytes // 4),), dtype=torch.float32, device=logits.device)
    if out is None:
        out = torch.empty((M,), dtype=torch.float32, device=logits.device)
    rc = lib().tbik_logsoftmax_gather_pmax(_ptr(logits), _ld(logits), _ptr(targets), _ptr(out),
                                           M, V, tp, _ptr(pmax), _ld(pmax), pmax.shape[1],
                                           _ptr(ws), ws.numel() * 4, _stream())
    _chk(rc, "tbik_logsoftmax_gather_pmax")
    return out, ws


def logsoftmax_shard_nodes(ws, M, tp):
    """View of the per-row shard partial sums inside a log-softmax workspace."""
    return ws[: M * tp].view(M, tp)


def tbik_softmax_causal(S, offset, scale, P=None):
    """S [B, Lq, Lk] fp32 -> P [B, Lq, Lk] bf16."""
    _need_gpu(S)
    B, Lq, Lk = S.shape
    if S.stride(2) != 1:
        raise ValueError("rows must be contiguous")
    if P is None:
        P = torch.empty((B, Lq, Lk), dtype=torch.bfloat16, device=S.device)
    rc = lib().tbik_softmax_causal(_ptr(S), S.stride(1), S.stride(0), _ptr(P), P.stride(1),
                                   P.stride(0), Lq, Lk, B, offset, float(scale), _stream())
    _chk(rc, "tbik_softmax_causal")
    return P


def tbik_primitive(op, x, y=None):
    _need_gpu(x)
    if y is None:
        y = torch.empty_like(x)
    rc = lib().tbik_primitive(op, _ptr(x), _ptr(y), x.numel(), _stream())
    _chk(rc, "tbik_primitive")
    return y


# --- training side -------------------------------------------------------------

def tbik_transpose_bf16(x, out=None):
    _bits(x); _need_gpu(x)
    rows, cols = x.shape
    if out is None:
        out = torch.empty((cols, rows), dtype=torch.bfloat16, device=x.device)
    rc = lib().tbik_transpose_bf16(_ptr(x), _ld(x), _ptr(out), _ld(out), rows, cols, _stream())
    _chk(rc, "tbik_transpose_bf16")
    return out


def _bytes_ws(nbytes, dev):
    return torch.empty((max(1, (nbytes + 15) // 16) * 4,), dtype=torch.float32, device=dev)


def tbik_gemm_dgrad(dY, W, leaf_mode=LEAF_MFMA, want_fp32=True, want_bf16=False, ws=None):
    """dX = dY W (tree over N): dY [M,N], W [N,K] -> (dX fp32 or None, dX bf16 or None)."""
    _bits(dY); _bits(W); _need_gpu(dY, W)
    M, N = dY.shape
    K = W.shape[1]
    dX = torch.empty((M, K), dtype=torch.float32, device=dY.device) if want_fp32 else None
    dXb = torch.empty((M, K), dtype=torch.bfloat16, device=dY.device) if want_bf16 else None
    need = lib().tbik_gemm_dgrad_workspace_bytes(M, N, K)
    if ws is None:
        ws = _bytes_ws(need, dY.device)
    rc = lib().tbik_gemm_dgrad(_ptr(dY), _ld(dY), _ptr(W), _ld(W), _ptr(dX), K, _ptr(dXb), M, N,
                               K, leaf_mode, _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _chk(rc, "tbik_gemm_dgrad")
    return dX, dXb


def tbik_gemm_wgrad(dY, X, dp=1, leaf_mode=LEAF_MFMA, ws=None, out=None):
    """dW = dY^T X (tree over the M/64 token leaves, dp simulated data-parallel
    shards): dY [M,N], X [M,K] -> (dW [N,K] fp32, shard partials [dp,N,K] or None)."""
    _bits(dY); _bits(X); _need_gpu(dY, X)
    M, N = dY.shape
    K = X.shape[1]
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=dY.device)
    need = lib().tbik_gemm_wgrad_workspace_bytes(M, N, K, dp)
    if ws is None:
        ws = _bytes_ws(need, dY.device)
    rc = lib().tbik_gemm_wgrad(_ptr(dY), _ld(dY), _ptr(X), _ld(X), _ptr(out), _ld(out), M, N, K, dp,
                               leaf_mode, _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _chk(rc, "tbik_gemm_wgrad")
    parts = None
    if dp > 1:
        r256 = lambda b: (b + 255) // 256 * 256
        off = (r256(N * M * 2) + r256(K * M * 2)) // 4
        parts = ws.view(torch.float32)[off:off + dp * N * K].view(dp, N, K)
    return out, parts


def tbik_rope_backward(dy, pos, cos_tab, sin_tab, dx=None):
    _bits(dy); _need_gpu(dy, pos, cos_tab, sin_tab)
    T, heads, d = dy.shape
    if dy.stride(2) != 1 or dy.stride(1) != d:
        raise ValueError("heads must be contiguous with stride head_dim")
    dx = _rows_like(dy) if dx is None else dx
    _same_rows(dx, dy, "dx")
    rc = lib().tbik_rope_backward(_ptr(dy), _ptr(dx), _ptr(pos), _ptr(cos_tab), _ptr(sin_tab), T,
                                  heads, d, dy.stride(0), cos_tab.shape[0], _stream())
    _chk(rc, "tbik_rope_backward")
    return dx


def tbik_swiglu_backward(gate, up, dout):
    """-> (dgate, dup) bf16."""
    _bits(gate); _bits(up); _bits(dout); _need_gpu(gate, up, dout)
    rows, cols = gate.shape
    dg = torch.empty((rows, cols), dtype=torch.bfloat16, device=gate.device)
    du = torch.empty_like(dg)
    rc = lib().tbik_swiglu_backward(_ptr(gate), _ptr(up), _ptr(dout), _ptr(dg), _ptr(du), rows,
                                    cols, _ld(gate), _ld(up), _ld(dout), _ld(dg), _ld(du),
                                    _stream())
    _chk(rc, "tbik_swiglu_backward")
    return dg, du


def tbik_rmsnorm_backward(x, r, w, dy, dr=None, eps=1e-6, dp=1, want_dw=True):
    """-> (dh bf16 [rows,H], dw fp32 [H] or None, shard nodes [dp,H] or None)."""
    _bits(x); _bits(r); _bits(w); _bits(dy); _need_gpu(x, r, w, dy)
    rows, H = x.shape
    ld = _ld(x)
    for t in (r, dy) + ((dr,) if dr is not None else ()):
        if _ld(t) != ld:
            raise ValueError("x, r, dy and dr must share the row stride")
    dh = _rows_like(x)
    dw = torch.empty((H,), dtype=torch.float32, device=x.device) if want_dw else None
    need = lib().tbik_rmsnorm_backward_workspace_bytes(rows, H, dp, int(want_dw))
    ws = torch.empty((max(1, need // 4),), dtype=torch.float32, device=x.device)
    rc = lib().tbik_rmsnorm_backward(_ptr(x), _ptr(r), _ptr(w), _ptr(dy), _ptr(dr), _ptr(dh),
                                     _ptr(dw), rows, H, ld, float(eps), dp, _ptr(ws), need,
                                     _stream())
    _chk(rc, "tbik_rmsnorm_backward")
    shards = None
    if want_dw:
        off = (rows + 63) // 64 * 64 + (rows // 64) * H
        shards = ws[off:off + dp * H].view(dp, H)
    return dh, dw, shards


# --- ceiling microbenchmarks --------------------------------------------------

def tbik_bench_mfma(seed, blocks, iters, out=None):
    """One launch of the matrix-core loop; seed: >= 2048 bytes on the device.
    Returns (out, flops of the launch)."""
    _need_gpu(seed)
    if out is None:
        out = torch.empty((blocks * 512,), dtype=torch.float32, device=seed.device)
    _chk(lib().tbik_bench_mfma(_ptr(seed), _ptr(out), blocks, iters, _stream()), "tbik_bench_mfma")
    return out, lib().tbik_bench_mfma_flops(blocks, iters)


def tbik_bench_hbm_read(buf, blocks, out=None):
    _need_gpu(buf)
    if out is None:
        out = torch.empty((blocks * 256,), dtype=torch.int32, device=buf.device)
    _chk(lib().tbik_bench_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), blocks,
                                   _stream()), "tbik_bench_hbm_read")
    return out


def tbik_bench_hbm_copy(src, dst, blocks):
    _need_gpu(src, dst)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst too small")
    _chk(lib().tbik_bench_hbm_copy(_ptr(src), _ptr(dst), n, blocks, _stream()),
         "tbik_bench_hbm_copy")
    return dst


def tbik_bench_copy_lds(buf, window_bytes, stages, blocks, out=None):
    """The GEMM ring's operand copy alone; returns (out, bytes moved)."""
    _need_gpu(buf)
    if window_bytes > buf.numel() * buf.element_size():
        raise ValueError("window larger than the buffer")
    if out is None:
        out = torch.empty((blocks * 512,), dtype=torch.int32, device=buf.device)
    _chk(lib().tbik_bench_copy_lds(_ptr(buf), window_bytes, stages, _ptr(out), blocks, _stream()),
         "tbik_bench_copy_lds")
    return out, blocks * stages * 32768
