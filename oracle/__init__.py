"""CPU oracle for the tree-based invariant kernels -- TEST INFRASTRUCTURE.

The slow scalar C implementation in ``tbik_oracle.c`` defines every result
the GPU library must reproduce.  This module only marshals numpy arrays into
it.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the GPU library never does.

Arrays of bf16 values are passed as ``numpy.uint16`` bit patterns.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        p = C.c_void_p
        i32, i64, f32, f64 = C.c_int, C.c_int64, C.c_float, C.c_double
        sig = {
            "or_bf16_to_f32": (f32, [C.c_uint16]),
            "or_f32_to_bf16": (C.c_uint16, [f32]),
            "or_tree_T": (i32, [i64]),
            "or_pair": (f32, [p, i64, p]),
            "or_tree": (f32, [p, i64, p]),
            "or_tree_sharded": (f32, [p, i64, i32, p, p]),
            "or_expf": (f32, [f32]),
            "or_logf": (f32, [f32]),
            "or_expf_array": (None, [p, p, i64]),
            "or_logf_array": (None, [p, p, i64]),
            "or_f32_to_bf16_array": (None, [p, p, i64]),
            "or_gemm": (i32, [p, i64, p, i64, p, i64, i32, i32, i32, i32]),
            "or_gemm_tpsim": (i32, [p, i64, p, i64, p, i64, i32, i32, i32, i32, p, i32]),
            "or_gemm_f64": (i32, [p, i64, p, i64, p, i64, i32, i32, i32, i32]),
            "or_gemm_naive_tp": (i32, [p, i64, p, i64, p, i64, i32, i32, i32, i32, i32]),
            "or_gemm_sampled": (i32, [p, i64, p, i64, i32, p, p, i64, p, i32]),
            "or_rmsnorm_residual": (None, [p, p, p, p, p, i32, i32, i64, f32, i32]),
            "or_rope_table": (None, [f64, i32, i32, p, p]),
            "or_rope": (None, [p, p, p, p, p, i32, i32, i32, i64, i32]),
            "or_swiglu": (None, [p, p, p, i32, i32, i64, i64, i64, i32]),
            "or_rope_backward": (None, [p, p, p, p, p, i32, i32, i32, i64]),
            "or_swiglu_backward": (None, [p, p, p, p, p, i32, i32, i64]),
            "or_rmsnorm_backward": (i32, [p, p, p, p, p, p, p, i32, i32, i64, f32, i32, p]),
            "or_logsoftmax_gather": (i32, [p, i64, p, p, i32, i32, i32, p]),
            "or_softmax_causal": (None, [p, i64, p, i64, i32, i32, i32, f32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _threads(n):
    """n, or by default the CPUs this process may use, at most 16 (one GPU's
    share of a host); threads split independent outputs, never a sum."""
    if n:
        return n
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(16, avail))


# --- primitives -------------------------------------------------------------

def bf16_to_f32(h):
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x):
    x = np.asarray(x, dtype=np.float32)
    shape = x.shape
    x = _c(x.ravel(), np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().or_f32_to_bf16_array(_ptr(x), _ptr(y), x.size)
    return y.reshape(shape)


def expf(x):
    x = _c(np.asarray(x, dtype=np.float32).ravel(), np.float32)
    y = np.empty_like(x)
    lib().or_expf_array(_ptr(x), _ptr(y), x.size)
    return y


def logf(x):
    x = _c(np.asarray(x, dtype=np.float32).ravel(), np.float32)
    y = np.empty_like(x)
    lib().or_logf_array(_ptr(x), _ptr(y), x.size)
    return y


def tree_T(n):
    return lib().or_tree_T(n)


def pair(v):
    v = _c(np.asarray(v, dtype=np.float32), np.float32)
    s = np.empty(max(1, v.size), np.float32)
    return np.float32(lib().or_pair(_ptr(v), v.size, _ptr(s)))


def tree(v):
    v = _c(np.asarray(v, dtype=np.float32), np.float32)
    s = np.empty(max(1, v.size), np.float32)
    return np.float32(lib().or_tree(_ptr(v), v.size, _ptr(s)))


def tree_sharded(v, tp):
    v = _c(np.asarray(v, dtype=np.float32), np.float32)
    s = np.empty(max(1, v.size), np.float32)
    nodes = np.zeros(8, np.float32)
    r = lib().or_tree_sharded(_ptr(v), v.size, tp, _ptr(s), _ptr(nodes))
    return np.float32(r), nodes[:tp].copy()


# --- GEMM -------------------------------------------------------------------

def gemm(A, W, nthreads=0):
    """A [M,K] uint16 (bf16), W [N,K] uint16 -> C [M,N] float32 (tree)."""
    A = _c(A, np.uint16); W = _c(W, np.uint16)
    M, K = A.shape; N = W.shape[0]
    C_ = np.empty((M, N), np.float32)
    rc = lib().or_gemm(_ptr(A), K, _ptr(W), K, _ptr(C_), N, M, N, K, _threads(nthreads))
    if rc:
        raise ValueError("oracle gemm: error %d" % rc)
    return C_


def gemm_tpsim(A, W, tp, nthreads=0):
    """Returns (C [M,N], partials [tp,M,N])."""
    A = _c(A, np.uint16); W = _c(W, np.uint16)
    M, K = A.shape; N = W.shape[0]
    C_ = np.empty((M, N), np.float32)
    ws = np.empty((tp, M, N), np.float32)
    rc = lib().or_gemm_tpsim(_ptr(A), K, _ptr(W), K, _ptr(C_), N, M, N, K, tp, _ptr(ws),
                             _threads(nthreads))
    if rc:
        raise ValueError("oracle gemm_tpsim: error %d" % rc)
    return C_, ws


def gemm_f64(A, W, nthreads=0):
    A = _c(A, np.uint16); W = _c(W, np.uint16)
    M, K = A.shape; N = W.shape[0]
    C_ = np.empty((M, N), np.float64)
    lib().or_gemm_f64(_ptr(A), K, _ptr(W), K, _ptr(C_), N, M, N, K, _threads(nthreads))
    return C_


def gemm_naive_tp(A, W, tp, nthreads=0):
    A = _c(A, np.uint16); W = _c(W, np.uint16)
    M, K = A.shape; N = W.shape[0]
    C_ = np.empty((M, N), np.float32)
    rc = lib().or_gemm_naive_tp(_ptr(A), K, _ptr(W), K, _ptr(C_), N, M, N, K, tp,
                                _threads(nthreads))
    if rc:
        raise ValueError("oracle naive tp: error %d" % rc)
    return C_


def gemm_sampled(A, W, rows, cols, nthreads=0):
    A = _c(A, np.uint16); W = _c(W, np.uint16)
    K = A.shape[1]
    rows = _c(np.asarray(rows, np.int32), np.int32)
    cols = _c(np.asarray(cols, np.int32), np.int32)
    out = np.empty(rows.size, np.float32)
    rc = lib().or_gemm_sampled(_ptr(A), A.shape[1], _ptr(W), W.shape[1], K, _ptr(rows),
                               _ptr(cols), rows.size, _ptr(out), _threads(nthreads))
    if rc:
        raise ValueError("oracle gemm_sampled: error %d" % rc)
    return out


# --- row reductions and elementwise nodes -----------------------------------

ROUNDING = {"once": 0, "each_op": 1}


def rmsnorm_residual(x, r, w, eps, rounding="once"):
    """rounding: "once" (fp32 intermediates) or "each_op" (bf16 after every op)."""
    x = _c(x, np.uint16); r = _c(r, np.uint16); w = _c(w, np.uint16)
    rows, H = x.shape
    y = np.empty_like(x); r_out = np.empty_like(x)
    lib().or_rmsnorm_residual(_ptr(x), _ptr(r), _ptr(w), _ptr(y), _ptr(r_out), rows, H, H,
                              np.float32(eps), ROUNDING[rounding])
    return y, r_out


def rope_table(theta, head_dim, max_pos):
    half = head_dim // 2
    c = np.empty((max_pos, half), np.float32)
    s = np.empty((max_pos, half), np.float32)
    lib().or_rope_table(float(theta), head_dim, max_pos, _ptr(c), _ptr(s))
    return c, s


def rope(x, pos, cos_tab, sin_tab, rounding="once"):
    """x [T, heads, head_dim] uint16."""
    x = _c(x, np.uint16)
    T, heads, hd = x.shape
    pos = _c(np.asarray(pos, np.int32), np.int32)
    cos_tab = _c(cos_tab, np.float32); sin_tab = _c(sin_tab, np.float32)
    y = np.empty_like(x)
    lib().or_rope(_ptr(x), _ptr(y), _ptr(pos), _ptr(cos_tab), _ptr(sin_tab), T, heads, hd,
                  heads * hd, ROUNDING[rounding])
    return y


def swiglu(g, u, rounding="once"):
    g = _c(g, np.uint16); u = _c(u, np.uint16)
    rows, cols = g.shape
    out = np.empty_like(g)
    lib().or_swiglu(_ptr(g), _ptr(u), _ptr(out), rows, cols, cols, cols, cols, ROUNDING[rounding])
    return out


def logsoftmax_gather(logits, targets, tp=1):
    """Returns (lp [M], shard_nodes [M, tp])."""
    logits = _c(logits, np.float32)
    M, V = logits.shape
    targets = _c(np.asarray(targets, np.int32), np.int32)
    out = np.empty(M, np.float32)
    nodes = np.empty((M, tp), np.float32)
    rc = lib().or_logsoftmax_gather(_ptr(logits), V, _ptr(targets), _ptr(out), M, V, tp,
                                    _ptr(nodes))
    if rc:
        raise ValueError("oracle logsoftmax: error %d" % rc)
    return out, nodes


def softmax_causal(S, offset, scale):
    S = _c(S, np.float32)
    Lq, Lk = S.shape
    P = np.empty((Lq, Lk), np.uint16)
    lib().or_softmax_causal(_ptr(S), Lk, _ptr(P), Lk, Lq, Lk, offset, np.float32(scale))
    return P


# --- training side: backward passes -------------------------------------------

def gemm_dgrad(dY, W, nthreads=0):
    """dX = dY W: dY [M,N], W [N,K] (uint16) -> [M,K] fp32, TREE over the N
    leaves (the GEMM with the weight transposed on the host)."""
    return gemm(dY, np.ascontiguousarray(np.asarray(W, np.uint16).T), nthreads)


def gemm_wgrad(dY, X, dp=1, nthreads=0):
    """dW = dY^T X: dY [M,N], X [M,K] -> ([N,K] fp32, partials [dp,N,K]);
    TREE over the M/64 token leaves, evaluated as dp data-parallel shards."""
    dYt = np.ascontiguousarray(np.asarray(dY, np.uint16).T)
    Xt = np.ascontiguousarray(np.asarray(X, np.uint16).T)
    return gemm_tpsim(dYt, Xt, dp, nthreads)


def rope_backward(dy, pos, cos_tab, sin_tab):
    """dy [T, heads, head_dim] uint16 -> dx (the rotation by -angle)."""
    dy = _c(dy, np.uint16)
    T, heads, hd = dy.shape
    pos = _c(np.asarray(pos, np.int32), np.int32)
    cos_tab = _c(cos_tab, np.float32); sin_tab = _c(sin_tab, np.float32)
    dx = np.empty_like(dy)
    lib().or_rope_backward(_ptr(dy), _ptr(dx), _ptr(pos), _ptr(cos_tab), _ptr(sin_tab), T, heads,
                           hd, heads * hd)
    return dx


def swiglu_backward(g, u, dout):
    """-> (dgate, dup) uint16."""
    g = _c(g, np.uint16); u = _c(u, np.uint16); dout = _c(dout, np.uint16)
    rows, cols = g.shape
    dg = np.empty_like(g); du = np.empty_like(g)
    lib().or_swiglu_backward(_ptr(g), _ptr(u), _ptr(dout), _ptr(dg), _ptr(du), rows, cols, cols)
    return dg, du


def rmsnorm_backward(x, r, w, dy, dr, eps, dp=1, want_dw=True):
    """-> (dh uint16 [rows,H], dw fp32 [H] or None, dw_shards [dp,H] or None)."""
    x = _c(x, np.uint16); r = _c(r, np.uint16); w = _c(w, np.uint16); dy = _c(dy, np.uint16)
    dr = None if dr is None else _c(dr, np.uint16)
    rows, H = x.shape
    dh = np.empty_like(x)
    dw = np.empty(H, np.float32) if want_dw else None
    shards = np.empty((dp, H), np.float32) if want_dw else None
    rc = lib().or_rmsnorm_backward(_ptr(x), _ptr(r), _ptr(w), _ptr(dy),
                                   None if dr is None else _ptr(dr), _ptr(dh),
                                   None if dw is None else _ptr(dw), rows, H, H,
                                   np.float32(eps), dp, None if shards is None else _ptr(shards))
    if rc:
        raise ValueError("oracle rmsnorm_backward: error %d" % rc)
    return dh, dw, shards
