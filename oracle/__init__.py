"""CPU oracle of the dropless MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The device library never imports it and it never
imports the device library; the two share only the seeded input generators.

The arithmetic lives in ``oracle.c`` (plain loops, fp64 accumulation, own
bf16 / E4M3 / E8M0 routines); this module marshals numpy arrays into it.
Function by function, the definitions and their sources are given in
``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (fp64, no contraction, OpenMP over rows)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i64, i32 = ctypes.c_int64, ctypes.c_int32
            sig = {
                "oracle_bf16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
                "oracle_f64_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
                "oracle_bf16_round_array": (None, [P, P, i64]),
                "oracle_e4m3_to_f64": (ctypes.c_double, [ctypes.c_uint8]),
                "oracle_f64_to_e4m3": (ctypes.c_uint8, [ctypes.c_double]),
                "oracle_e8m0_to_f64": (ctypes.c_double, [ctypes.c_uint8]),
                "oracle_route_logits": (None, [P, P, P, i64, i32, i32, P]),
                "oracle_route_topk": (None, [P, i64, i32, i32, i32, P, P]),
                "oracle_permute": (None, [P, i64, i32, i32, P, P, P, P]),
                "oracle_gather_rows": (None, [P, P, i64, i32, i32, P]),
                "oracle_grouped_gemm_rows": (None, [P, P, P, i32, i32, i32, P, i64, P]),
                "oracle_gemm_swiglu_rows": (None, [P, P, P, i32, i32, i32, P, i64, P, P]),
                "oracle_unpermute_combine": (None, [P, P, P, i64, i32, i32, P]),
                "oracle_mxfp8_quantize_rows": (None, [P, i64, i32, P, P]),
                "oracle_mxfp8_quantize_cols_grouped": (None, [P, i64, i32, P, i32, P, P]),
                "oracle_mx_grouped_gemm_rows": (None, [P, P, P, P, P, i32, i32, i32, i32, P, i64, P]),
                "oracle_combine_backward": (None, [P, P, P, P, i64, i32, i32, P, P]),
                "oracle_swiglu_backward": (None, [P, P, i64, i32, P]),
                "oracle_grouped_dgrad_rows": (None, [P, P, P, i32, i32, i32, P, i64, P]),
                "oracle_grouped_wgrad": (None, [P, P, P, i32, i32, i32, P, i32, P]),
                "oracle_mx_grouped_wgrad": (None, [P, P, P, P, P, i32, i32, i32, P]),
                "oracle_e2m1_to_f64": (ctypes.c_double, [ctypes.c_uint8]),
                "oracle_f64_to_e2m1": (ctypes.c_uint8, [ctypes.c_double]),
                "oracle_mxfp4_quantize_rows": (None, [P, i64, i32, P, P]),
                "oracle_mx4_grouped_gemm_rows": (None, [P, P, P, P, P, i32, i32, i32, i32, P, i64, P]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


# --------------------------------------------------------------------------
# marshalling helpers: bf16 tensors travel as uint16 bit patterns
# --------------------------------------------------------------------------

def u16(a) -> np.ndarray:
    """bf16 torch tensor / uint16 array -> contiguous uint16 numpy array."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            assert a.dtype == torch.bfloat16, a.dtype
            return a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _np(a, dtype) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def bf16_to_f64(a) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    b = u16(a).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_round_array(_p(v), _p(out), v.size)
    return out


def e4m3_to_f64(codes) -> np.ndarray:
    L = lib()
    c = _np(codes, np.uint8)
    table = np.array([L.oracle_e4m3_to_f64(i) for i in range(256)], dtype=np.float64)
    return table[c]


def e8m0_to_f64(s) -> np.ndarray:
    """E8M0 scale bytes -> 2^(s-127); 0xFF -> NaN."""
    L = lib()
    table = np.array([L.oracle_e8m0_to_f64(i) for i in range(256)], dtype=np.float64)
    return table[_np(s, np.uint8)]


def f64_to_e4m3(v) -> np.ndarray:
    L = lib()
    v = np.ascontiguousarray(v, dtype=np.float64)
    return np.array([L.oracle_f64_to_e4m3(float(x)) for x in v.ravel()], dtype=np.uint8).reshape(v.shape)


# --------------------------------------------------------------------------
# the layer, step by step
# --------------------------------------------------------------------------

def route_logits(x, w_router, bias=None) -> np.ndarray:
    """Router scores in fp64: x [T,d] bf16, w_router [E,d] bf16, bias fp32 [E] or None -> [T,E]."""
    xs, ws = u16(x), u16(w_router)
    T, d = xs.shape
    E = ws.shape[0]
    assert ws.shape[1] == d
    b = None if bias is None else _np(bias, np.float32)
    out = np.empty((T, E), np.float64)
    lib().oracle_route_logits(_p(xs), _p(ws), _p(b), T, d, E, _p(out))
    return out


def route_topk(logits, K: int, renormalize: bool = True):
    """-> ids int32 [T,K], w fp32 [T,K]."""
    l = _np(logits, np.float32)
    T, E = l.shape
    assert 1 <= K <= E <= 1024
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    lib().oracle_route_topk(_p(l), T, E, K, int(bool(renormalize)), _p(ids), _p(w))
    return ids, w


def permute(ids, E: int):
    """-> group_sizes [E], group_offsets [E+1], perm_src [M], perm_dst [T*K] (int32)."""
    ids = _np(ids, np.int32)
    T, K = ids.shape
    assert ids.size == 0 or (ids.min() >= 0 and ids.max() < E)
    sizes = np.empty(E, np.int32)
    offs = np.empty(E + 1, np.int32)
    src = np.empty(T * K, np.int32)
    dst = np.empty(T * K, np.int32)
    lib().oracle_permute(_p(ids), T, E, K, _p(sizes), _p(offs), _p(src), _p(dst))
    return sizes, offs, src, dst


def gather_rows(x, perm_src, K: int) -> np.ndarray:
    xs = u16(x)
    src = _np(perm_src, np.int32)
    T, d = xs.shape
    out = np.empty((src.size, d), np.uint16)
    lib().oracle_gather_rows(_p(xs), _p(src), src.size, d, K, _p(out))
    return out


def _rows(rows, M: int) -> np.ndarray:
    return np.arange(M, dtype=np.int64) if rows is None else _np(rows, np.int64)


def grouped_gemm(A, B, group_sizes, rows=None) -> np.ndarray:
    """C[r] = bf16(A[r] @ B[e(r)]^T) for the given rows (default all) -> uint16 [nrows, N]."""
    a, b, s = u16(A), u16(B), _np(group_sizes, np.int32)
    G, N, Kd = b.shape
    assert a.shape[1] == Kd and s.size == G
    r = _rows(rows, int(s.sum()))
    out = np.zeros((r.size, N), np.uint16)
    lib().oracle_grouped_gemm_rows(_p(a), _p(b), _p(s), G, N, Kd, _p(r), r.size, _p(out))
    return out


def gemm_swiglu(A, W1p, group_sizes, rows=None, keep_gu: bool = False):
    """h[r] = bf16(silu(g) * u), [g|u] = A[r] @ W1p[e]^T -> (h [nrows,f], gu [nrows,2f] or None)."""
    a, b, s = u16(A), u16(W1p), _np(group_sizes, np.int32)
    G, N2, Kd = b.shape
    f = N2 // 2
    assert a.shape[1] == Kd and s.size == G
    r = _rows(rows, int(s.sum()))
    h = np.zeros((r.size, f), np.uint16)
    gu = np.zeros((r.size, 2 * f), np.uint16) if keep_gu else None
    lib().oracle_gemm_swiglu_rows(_p(a), _p(b), _p(s), G, f, Kd, _p(r), r.size, _p(h), _p(gu))
    return h, gu


def unpermute_combine(y_perm, w, perm_dst, T: int, K: int) -> np.ndarray:
    yp = u16(y_perm)
    dst = _np(perm_dst, np.int32)
    wv = None if w is None else _np(w, np.float32)
    d = yp.shape[1]
    y = np.empty((T, d), np.uint16)
    lib().oracle_unpermute_combine(_p(yp), _p(wv), _p(dst), T, d, K, _p(y))
    return y


def mxfp8_quantize(x, axis: int = 0, group_sizes=None):
    """axis 0: 32-blocks along columns -> (codes [R,C] uint8, scales [R,C/32] uint8).
    axis 1: 32-blocks down columns restarting at each group -> scales [sum ceil(s/32), C]."""
    xs = u16(x)
    R, C = xs.shape
    q = np.zeros((R, C), np.uint8)
    if axis == 0:
        assert C % 32 == 0
        s = np.empty((R, C // 32), np.uint8)
        lib().oracle_mxfp8_quantize_rows(_p(xs), R, C, _p(q), _p(s))
        return q, s
    g = _np(group_sizes, np.int32)
    assert int(g.sum()) <= R
    nb = int(((g.astype(np.int64) + 31) // 32).sum())
    s = np.zeros((nb, C), np.uint8)
    lib().oracle_mxfp8_quantize_cols_grouped(_p(xs), R, C, _p(g), g.size, _p(q), _p(s))
    return q, s


def mx_grouped_gemm(Aq, As, Bq, Bs, group_sizes, swiglu: bool = False, rows=None) -> np.ndarray:
    aq, as_, bq, bs = (_np(t, np.uint8) for t in (Aq, As, Bq, Bs))
    s = _np(group_sizes, np.int32)
    G, N, Kd = bq.shape
    r = _rows(rows, int(s.sum()))
    nout = N // 2 if swiglu else N
    out = np.zeros((r.size, nout), np.uint16)
    lib().oracle_mx_grouped_gemm_rows(_p(aq), _p(as_), _p(bq), _p(bs), _p(s), G, N, Kd, int(swiglu),
                                      _p(r), r.size, _p(out))
    return out


def e2m1_to_f64(codes) -> np.ndarray:
    L = lib()
    c = _np(codes, np.uint8)
    table = np.array([L.oracle_e2m1_to_f64(i) for i in range(16)], dtype=np.float64)
    return table[c & 15]


def f64_to_e2m1(v) -> np.ndarray:
    L = lib()
    v = np.ascontiguousarray(v, dtype=np.float64)
    return np.array([L.oracle_f64_to_e2m1(float(x)) for x in v.ravel()], dtype=np.uint8).reshape(v.shape)


def mxfp4_quantize(x):
    """32-blocks along columns -> (codes [R,C] uint8, one E2M1 code per byte; scales [R,C/32] uint8)."""
    xs = u16(x)
    R, C = xs.shape
    assert C % 32 == 0
    q = np.empty((R, C), np.uint8)
    s = np.empty((R, C // 32), np.uint8)
    lib().oracle_mxfp4_quantize_rows(_p(xs), R, C, _p(q), _p(s))
    return q, s


def mx4_grouped_gemm(Aq, As, Bq, Bs, group_sizes, swiglu: bool = False, rows=None) -> np.ndarray:
    """Codes one per byte: Aq [M,K], Bq [G,N,K]; scales [M,K/32], [G,N,K/32]."""
    aq, as_, bq, bs = (_np(t, np.uint8) for t in (Aq, As, Bq, Bs))
    s = _np(group_sizes, np.int32)
    G, N, Kd = bq.shape
    r = _rows(rows, int(s.sum()))
    nout = N // 2 if swiglu else N
    out = np.zeros((r.size, nout), np.uint16)
    lib().oracle_mx4_grouped_gemm_rows(_p(aq), _p(as_), _p(bq), _p(bs), _p(s), G, N, Kd, int(swiglu),
                                       _p(r), r.size, _p(out))
    return out


def mx_grouped_wgrad(Aq, As, Bq, Bs, group_sizes) -> np.ndarray:
    """C[e] = bf16(sum over group e's rows of a[r]^T b[r]) -> [G, P, Q], from
    operands quantised by mxfp8_quantize(axis=1) (codes [rows, P|Q], scales
    [sum ceil(s/32), P|Q])."""
    aq, as_, bq, bs = (_np(t, np.uint8) for t in (Aq, As, Bq, Bs))
    s = _np(group_sizes, np.int32)
    P, Q = aq.shape[1], bq.shape[1]
    out = np.zeros((s.size, P, Q), np.uint16)
    lib().oracle_mx_grouped_wgrad(_p(aq), _p(as_), _p(bq), _p(bs), _p(s), s.size, P, Q, _p(out))
    return out


def combine_backward(dy, y_perm, w, perm_dst, K: int):
    """-> dy_perm bf16 [M,d], dw fp32 [T,K]."""
    g, yp = u16(dy), u16(y_perm)
    wv = _np(w, np.float32)
    dst = _np(perm_dst, np.int32)
    T, d = g.shape
    dyp = np.zeros(yp.shape, np.uint16)
    dw = np.empty((T, K), np.float32)
    lib().oracle_combine_backward(_p(g), _p(yp), _p(wv), _p(dst), T, d, K, _p(dyp), _p(dw))
    return dyp, dw


def swiglu_backward(gu, dh) -> np.ndarray:
    a, b = u16(gu), u16(dh)
    M, f = b.shape
    out = np.empty((M, 2 * f), np.uint16)
    lib().oracle_swiglu_backward(_p(a), _p(b), M, f, _p(out))
    return out


def grouped_dgrad(dC, B, group_sizes, rows=None) -> np.ndarray:
    """dA[r] = bf16(dC[r] @ B[e(r)]) for C = A @ B[e]^T."""
    g, b, s = u16(dC), u16(B), _np(group_sizes, np.int32)
    G, N, Kd = b.shape
    r = _rows(rows, int(s.sum()))
    out = np.zeros((r.size, Kd), np.uint16)
    lib().oracle_grouped_dgrad_rows(_p(g), _p(b), _p(s), G, N, Kd, _p(r), r.size, _p(out))
    return out


def grouped_wgrad(dC, A, group_sizes, groups: Optional[Sequence[int]] = None) -> np.ndarray:
    """dB[e] = bf16(sum over the group's rows of dC[r]^T A[r]) -> [ngroups, N, Kd]."""
    g, a, s = u16(dC), u16(A), _np(group_sizes, np.int32)
    N, Kd = g.shape[1], a.shape[1]
    G = s.size
    gl = None if groups is None else np.ascontiguousarray(groups, dtype=np.int32)
    ng = G if gl is None else gl.size
    out = np.zeros((ng, N, Kd), np.uint16)
    lib().oracle_grouped_wgrad(_p(g), _p(a), _p(s), G, N, Kd, _p(gl), ng, _p(out))
    return out


# --------------------------------------------------------------------------
# whole-layer compositions
# --------------------------------------------------------------------------

def layer_forward(logits, x, w1p, w2, K: int, keep: bool = False):
    """Route -> permute -> GEMM+SwiGLU -> GEMM -> combine.  Returns y (uint16
    [T,d]) and, if keep, a dict of every intermediate."""
    ids, w = route_topk(logits, K)
    E = int(w1p.shape[0])
    sizes, offs, src, dst = permute(ids, E)
    xp = gather_rows(x, src, K)
    h, gu = gemm_swiglu(xp, w1p, sizes, keep_gu=keep)
    yp = grouped_gemm(h, w2, sizes)
    T = ids.shape[0]
    y = unpermute_combine(yp, w, dst, T, K)
    if not keep:
        return y, None
    return y, dict(ids=ids, w=w, sizes=sizes, offs=offs, perm_src=src, perm_dst=dst,
                   x_perm=xp, h=h, gu=gu, y_perm=yp)


def layer_backward(dy, saved, w1p, w2, K: int):
    """Backward of layer_forward given its kept intermediates."""
    sizes, dst = saved["sizes"], saved["perm_dst"]
    dyp, dw = combine_backward(dy, saved["y_perm"], saved["w"], dst, K)
    dh = grouped_dgrad(dyp, w2, sizes)
    dw2 = grouped_wgrad(dyp, saved["h"], sizes)
    dgu = swiglu_backward(saved["gu"], dh)
    dxp = grouped_dgrad(dgu, w1p, sizes)
    dw1p = grouped_wgrad(dgu, saved["x_perm"], sizes)
    T = saved["ids"].shape[0]
    dx = unpermute_combine(dxp, None, dst, T, K)
    return dict(dy_perm=dyp, dw=dw, dh=dh, dw2=dw2, dgu=dgu, dx_perm=dxp, dw1p=dw1p, dx=dx)


# --------------------------------------------------------------------------
# the layer in MXFP8 (blog: group-aware MXFP8 quantisation; "Optimization 1":
# MXFP8 block scaling of the expert matmuls), composed of the functions above
# --------------------------------------------------------------------------

def _quant_experts(w, axis: int):
    """[E, R, C] bf16 -> codes and scales per expert: axis 0 -> ([E, R, C],
    [E, R, C/32]) blocks along C; axis 1 -> ([E, C, R], [E, C, R/32]) blocks
    down R, each column's codes contiguous (the weight operand of a data
    gradient, contracted over R)."""
    wb = u16(w)
    E, R, C = wb.shape
    if axis == 0:
        q, s = mxfp8_quantize(wb.reshape(E * R, C), 0)
        return q.reshape(E, R, C), s.reshape(E, R, C // 32)
    qs, ss = [], []
    for e in range(E):
        q, s = mxfp8_quantize(wb[e], 1, np.array([R], np.int32))
        qs.append(q.T.copy())
        ss.append(s.T.copy())
    return np.stack(qs), np.stack(ss)


def layer_forward_mxfp8(logits, x, w1p, w2, K: int):
    """layer_forward with MXFP8 GEMMs: the permuted rows and h quantised along
    their rows (axis 0), the weights along their contraction; h from the
    gate/up accumulators, the pre-activations kept in bf16."""
    ids, w = route_topk(logits, K)
    E = int(w1p.shape[0])
    sizes, offs, src, dst = permute(ids, E)
    xp = gather_rows(x, src, K)
    xq, xs = mxfp8_quantize(xp, 0)
    w1q, w1s = _quant_experts(w1p, 0)
    gu = mx_grouped_gemm(xq, xs, w1q, w1s, sizes)
    h = mx_grouped_gemm(xq, xs, w1q, w1s, sizes, swiglu=True)
    hq, hs = mxfp8_quantize(h, 0)
    w2q, w2s = _quant_experts(w2, 0)
    yp = mx_grouped_gemm(hq, hs, w2q, w2s, sizes)
    T = ids.shape[0]
    y = unpermute_combine(yp, w, dst, T, K)
    return y, dict(ids=ids, w=w, sizes=sizes, offs=offs, perm_src=src, perm_dst=dst, x_perm=xp, h=h, gu=gu,
                   y_perm=yp)


def layer_backward_mxfp8(dy, saved, w1p, w2, K: int):
    """layer_backward with MXFP8 GEMMs: a data gradient quantises its left
    operand along the contraction (axis 0) and the weight down its output
    axis; a weight gradient quantises both operands down the tokens, blocks
    restarting at every expert's rows (group-aware, axis 1)."""
    sizes, dst = saved["sizes"], saved["perm_dst"]
    dyp, dw = combine_backward(dy, saved["y_perm"], saved["w"], dst, K)
    q, s = mxfp8_quantize(dyp, 0)
    w2tq, w2ts = _quant_experts(w2, 1)
    dh = mx_grouped_gemm(q, s, w2tq, w2ts, sizes)
    aq, as_ = mxfp8_quantize(dyp, 1, sizes)
    bq, bs = mxfp8_quantize(saved["h"], 1, sizes)
    dw2 = mx_grouped_wgrad(aq, as_, bq, bs, sizes)
    dgu = swiglu_backward(saved["gu"], dh)
    q, s = mxfp8_quantize(dgu, 0)
    w1tq, w1ts = _quant_experts(w1p, 1)
    dxp = mx_grouped_gemm(q, s, w1tq, w1ts, sizes)
    aq, as_ = mxfp8_quantize(dgu, 1, sizes)
    bq, bs = mxfp8_quantize(saved["x_perm"], 1, sizes)
    dw1p = mx_grouped_wgrad(aq, as_, bq, bs, sizes)
    T = saved["ids"].shape[0]
    dx = unpermute_combine(dxp, None, dst, T, K)
    return dict(dy_perm=dyp, dw=dw, dh=dh, dw2=dw2, dgu=dgu, dx_perm=dxp, dw1p=dw1p, dx=dx)
