"""ctypes binding of the fp64 CPU oracle (``libswinoracle.so``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU baseline leg of the benchmark.  The product path never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# a sanitizer build of the oracle may be substituted (tests/test_sanitizers.py)
LIB_PATH = os.environ.get("SWIN_ORACLE_LIB") or os.path.join(_HERE, "libswinoracle.so")
_SRC = os.path.join(_HERE, "swin_oracle.c")

F64, F32, BF16 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compiles the oracle with gcc; returns the library path."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                        "-o", tmp, _SRC, "-lm", "-lpthread"], check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I, L64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_long
        L.oracle_roll.argtypes = [P, I, I, I, I, I, I, P]
        L.oracle_window_partition.argtypes = [P, I, I, I, I, I, P]
        L.oracle_window_reverse.argtypes = [P, I, I, I, I, I, P]
        L.oracle_rel_index.argtypes = [I, P]
        L.oracle_region_labels.argtypes = [I, I, I, I, P]
        L.oracle_shift_mask.argtypes = [I, I, I, I, P]
        L.oracle_window_attention.argtypes = [P, P, P, L64, I, I, I, I, I, I, P]
        L.oracle_window_attention.restype = I
        L.oracle_swin_wattn_fwd.argtypes = [P, I, P, I, I, I, I, I, I, I, I, I, P]
        L.oracle_swin_wattn_fwd.restype = I
        L.oracle_swin_wattn_windows.argtypes = [P, I, P, I, I, I, I, I, I, I, L64, P, I, P, P]
        L.oracle_swin_wattn_windows.restype = I
        L.oracle_linear.argtypes = [P, I, L64, I, P, I, I, P, P, I, I, P]
        L.oracle_linear.restype = I
        L.oracle_layernorm.argtypes = [P, I, L64, I, P, P, ctypes.c_double, P]
        L.oracle_layernorm.restype = I
        L.oracle_swin_wattn_bwd.argtypes = [P, I, P, P, I, I, I, I, I, I, I, I, I, P, P]
        L.oracle_swin_wattn_bwd.restype = I
        L.oracle_dequant_qkv_i8.argtypes = [P, L64, I, P, P]
        L.oracle_linear_i8.argtypes = [P, L64, I, ctypes.c_float, P, I, P, P, P, I, P, I, P, P, P]
        L.oracle_linear_i8.restype = I
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def roll(x, sy: int, sx: int) -> np.ndarray:
    x = _f64(x)
    B, H, W, C = x.shape
    y = np.empty_like(x)
    lib().oracle_roll(_ptr(x), B, H, W, C, sy, sx, _ptr(y))
    return y


def window_partition(x, M: int) -> np.ndarray:
    x = _f64(x)
    B, H, W, C = x.shape
    win = np.empty((B, H // M, W // M, M * M, C), dtype=np.float64)
    lib().oracle_window_partition(_ptr(x), B, H, W, C, M, _ptr(win))
    return win


def window_reverse(win, H: int, W: int, M: int) -> np.ndarray:
    win = _f64(win)
    B, C = win.shape[0], win.shape[-1]
    x = np.empty((B, H, W, C), dtype=np.float64)
    lib().oracle_window_reverse(_ptr(win), B, H, W, C, M, _ptr(x))
    return x


def rel_index(M: int) -> np.ndarray:
    out = np.empty((M * M, M * M), dtype=np.int32)
    lib().oracle_rel_index(M, _ptr(out))
    return out


def region_labels(H: int, W: int, M: int, s: int) -> np.ndarray:
    out = np.empty((H, W), dtype=np.int32)
    lib().oracle_region_labels(H, W, M, s, _ptr(out))
    return out


def shift_mask(H: int, W: int, M: int, s: int) -> np.ndarray:
    out = np.empty(((H // M) * (W // M), M * M, M * M), dtype=np.float64)
    lib().oracle_shift_mask(H, W, M, s, _ptr(out))
    return out


def window_attention(win_qkv, table, mask, M: int, heads: int, head_dim: int,
                     npad: int = 0, nthreads: int = 0) -> np.ndarray:
    """``win_qkv [nWin, N, 3, heads, head_dim]`` -> ``[nWin, N, heads*head_dim]``."""
    win_qkv = _f64(win_qkv)
    table = np.ascontiguousarray(table, dtype=np.float32)
    nWin = win_qkv.shape[0]
    N = M * M
    if mask is not None:
        mask = _f64(mask)
        nW = mask.shape[0]
        mptr = _ptr(mask)
    else:
        nW, mptr = 1, None
    out = np.empty((nWin, N, heads * head_dim), dtype=np.float64)
    lib().oracle_window_attention(_ptr(win_qkv), _ptr(table), mptr, nWin, nW, M, heads,
                                  head_dim, npad, nthreads, _ptr(out))
    return out


def _qkv_arg(qkv):
    if qkv.dtype == np.uint16:
        return np.ascontiguousarray(qkv), BF16
    if qkv.dtype == np.float32:
        return np.ascontiguousarray(qkv), F32
    return _f64(qkv), F64


def swin_wattn_fwd(qkv, table, window: int, shift: int, npad: int = 0,
                   nthreads: int = 0, return_threads: bool = False):
    """Whole forward.  ``qkv [B,H,W,3,heads,head_dim]`` (uint16 = bfloat16
    patterns, float32 or float64); returns float64 ``[B,H,W,heads*head_dim]``."""
    q, code = _qkv_arg(qkv)
    B, H, W, three, nh, d = q.shape
    assert three == 3
    table = np.ascontiguousarray(table, dtype=np.float32)
    out = np.empty((B, H, W, nh * d), dtype=np.float64)
    used = lib().oracle_swin_wattn_fwd(_ptr(q), code, _ptr(table), B, H, W, nh, d, window,
                                       shift, npad, nthreads, _ptr(out))
    if used < 0:
        raise ValueError("oracle rejected the arguments")
    return (out, used) if return_threads else out


def swin_wattn_windows(qkv, table, window: int, shift: int, sel, nthreads: int = 0):
    """Forward of selected windows ``sel`` (ids ``b*nW + w``).

    Returns ``(out [nsel, N, C] float64, pos [nsel, N] int64)`` where ``pos`` is
    the flattened image position ``(b*H + y)*W + x`` of every token."""
    q, code = _qkv_arg(qkv)
    B, H, W, three, nh, d = q.shape
    table = np.ascontiguousarray(table, dtype=np.float32)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    N = window * window
    out = np.empty((len(sel), N, nh * d), dtype=np.float64)
    pos = np.empty((len(sel), N), dtype=np.int64)
    used = lib().oracle_swin_wattn_windows(_ptr(q), code, _ptr(table), B, H, W, nh, d, window,
                                           shift, len(sel), _ptr(sel), nthreads, _ptr(out),
                                           _ptr(pos))
    if used < 0:
        raise ValueError("oracle rejected the arguments")
    return out, pos


def linear(x, w, bias=None, residual=None, nthreads: int = 0, return_threads: bool = False):
    """``y = x @ w.T + bias (+ residual)`` in fp64.  ``x [..., K]``, ``w [N, K]``
    (uint16 = bfloat16 patterns, float32 or float64), ``bias [N]`` float32,
    ``residual [..., N]``.  Returns float64 ``[..., N]``."""
    xq, xc = _qkv_arg(x)
    wq, wc = _qkv_arg(w)
    N, K = wq.shape
    assert xq.shape[-1] == K
    lead = xq.shape[:-1]
    T = int(np.prod(lead)) if lead else 1
    bp = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (N,)
        bp = _ptr(bias)
    rp, rc = None, F64
    if residual is not None:
        rq, rc = _qkv_arg(residual)
        assert rq.shape == lead + (N,)
        rp = _ptr(rq)
    y = np.empty(lead + (N,), dtype=np.float64)
    used = lib().oracle_linear(_ptr(xq), xc, T, K, _ptr(wq), wc, N, bp, rp, rc, nthreads, _ptr(y))
    if used < 0:
        raise ValueError("oracle rejected the arguments")
    return (y, used) if return_threads else y


def layernorm(x, gamma, beta, eps: float = 1e-5):
    """Layer normalisation over the last dimension in fp64.  ``x [..., C]``
    (uint16 = bfloat16 patterns, float32 or float64); ``gamma, beta [C]``
    float32.  Returns float64 ``[..., C]``."""
    xq, xc = _qkv_arg(x)
    C = xq.shape[-1]
    T = int(np.prod(xq.shape[:-1])) if xq.ndim > 1 else 1
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    assert gamma.shape == (C,) and beta.shape == (C,)
    y = np.empty(xq.shape, dtype=np.float64)
    if lib().oracle_layernorm(_ptr(xq), xc, T, C, _ptr(gamma), _ptr(beta), eps, _ptr(y)) < 0:
        raise ValueError("oracle rejected the arguments")
    return y


def swin_wattn_bwd(qkv, table, dout, window: int, shift: int, nthreads: int = 0,
                   return_threads: bool = False):
    """Backward of the whole forward.  ``qkv [B,H,W,3,heads,head_dim]``,
    ``dout [B,H,W,heads*head_dim]`` (uint16 = bfloat16 patterns, float32 or
    float64), ``table`` float32.  Returns float64 ``(dqkv [B,H,W,3,heads,
    head_dim], dtable [(2*window-1)**2, heads])``."""
    q, code = _qkv_arg(qkv)
    g, gcode = _qkv_arg(dout)
    B, H, W, three, nh, d = q.shape
    assert three == 3 and g.shape == (B, H, W, nh * d)
    table = np.ascontiguousarray(table, dtype=np.float32)
    dq = np.empty(q.shape, dtype=np.float64)
    dt = np.empty(table.shape, dtype=np.float64)
    used = lib().oracle_swin_wattn_bwd(_ptr(q), code, _ptr(table), _ptr(g), gcode, B, H, W, nh, d,
                                       window, shift, nthreads, _ptr(dq), _ptr(dt))
    if used < 0:
        raise ValueError("oracle rejected the arguments")
    return (dq, dt, used) if return_threads else (dq, dt)


def dequant_qkv_i8(codes, scales) -> np.ndarray:
    """INT8 q, k, v codes ``[..., 3, heads, head_dim]`` (int8) times one
    scale per part (query, key, value); returns float64 of the same shape."""
    c = np.ascontiguousarray(codes, dtype=np.int8)
    assert c.ndim >= 3 and c.shape[-3] == 3
    C = c.shape[-2] * c.shape[-1]
    tokens = c.size // (3 * C)
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    assert sc.shape == (3,)
    out = np.empty(c.shape, dtype=np.float64)
    lib().oracle_dequant_qkv_i8(_ptr(c), tokens, C, _ptr(sc), _ptr(out))
    return out


def swin_wattn_fwd_i8(codes, scales, table, window: int, shift: int, nthreads: int = 0,
                      return_threads: bool = False):
    """The forward of INT8 q, k, v: the fp64 forward of the dequantized
    codes.  ``codes [B,H,W,3,heads,head_dim]`` int8, ``scales`` (query, key,
    value) float32."""
    return swin_wattn_fwd(dequant_qkv_i8(codes, scales), table, window, shift,
                          nthreads=nthreads, return_threads=return_threads)


def linear_i8(xq, sx: float, wq, sw, bias=None, residual=None, so=None, nthreads: int = 0,
              return_threads: bool = False):
    """INT8 linear layer.  ``xq [..., K]`` int8 codes with scale ``sx``;
    ``wq [N, K]`` int8 codes with per-output-channel scales ``sw [N]``;
    ``bias [N]`` float32; ``residual [..., N]`` (uint16 = bfloat16
    patterns, float32 or float64); ``so [N]`` output scales for INT8 output
    (no residual then).  Returns ``(acc int64, y float64, yq int8 or None)``:
    the exact integer sums, the dequantized value and the output codes."""
    x = np.ascontiguousarray(xq, dtype=np.int8)
    w = np.ascontiguousarray(wq, dtype=np.int8)
    N, K = w.shape
    assert x.shape[-1] == K
    lead = x.shape[:-1]
    T = int(np.prod(lead)) if lead else 1
    swa = np.ascontiguousarray(sw, dtype=np.float32)
    assert swa.shape == (N,)
    bp = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (N,)
        bp = _ptr(bias)
    rp, rc = None, F64
    if residual is not None:
        rq, rc = _qkv_arg(residual)
        assert rq.shape == lead + (N,)
        rp = _ptr(rq)
    sop, yq = None, None
    if so is not None:
        so = np.ascontiguousarray(so, dtype=np.float32)
        assert so.shape == (N,)
        sop = so.ctypes.data_as(ctypes.c_void_p)
        yq = np.empty(lead + (N,), dtype=np.int8)
    acc = np.empty(lead + (N,), dtype=np.int64)
    y = np.empty(lead + (N,), dtype=np.float64)
    used = lib().oracle_linear_i8(_ptr(x), T, K, float(sx), _ptr(w), N, _ptr(swa), bp, rp, rc, sop,
                                  nthreads, _ptr(acc), _ptr(y), None if yq is None else _ptr(yq))
    if used < 0:
        raise ValueError("oracle rejected the arguments")
    return ((acc, y, yq), used) if return_threads else (acc, y, yq)
