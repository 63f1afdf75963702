"""Python binding of libswinattn: fused shifted-window multi-head attention
forward (Swin Transformer) for MI355X.

Argument marshalling only: every function forwards to the C ABI declared in
``include/swinattn.h`` under the same name and returns its integer status.
Tensors may be passed as torch tensors (their ``data_ptr()`` is used) or as
raw device addresses.  ``stream=None`` means torch's current stream when torch
has a GPU, else the null stream.  There is no fallback: importing this package
fails if ``libswinattn.so`` has not been built (``python
shifted_window_attention_swin_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

try:  # load torch first so that its HIP runtime is the one this library binds to
    import torch as _torch
except Exception:  # pragma: no cover - torch is optional for the binding itself
    _torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswinattn.so")

SWIN_OK = 0
SWIN_ERR_INVALID_ARG = -1
SWIN_ERR_UNSUPPORTED = -2
SWIN_ERR_NOT_PREPARED = -3
SWIN_ERR_HIP = -4

EXPORTS = ("swin_wattn_precompute", "swin_wattn_fwd", "swin_wattn_fwd_f32", "swin_wattn_fwd_i8",
           "swin_wattn_bwd",
           "swin_wattn_copy_index", "swin_wattn_copy_mask", "swin_wattn_copy_region",
           "swin_linear_pack_weight", "swin_linear_fwd", "swin_linear_i8_pack_weight",
           "swin_linear_i8_fwd", "swin_ln_linear_pack_weight",
           "swin_ln_linear_fwd", "swin_ln_qkv_wattn_fwd",
           "swin_wattn_release", "swin_wattn_status_string")


class SwinAttnError(RuntimeError):
    def __init__(self, status: int, call: str = ""):
        self.status = status
        super().__init__(f"{call}: {swin_wattn_status_string(status)}" if call
                         else swin_wattn_status_string(status))


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python shifted_window_attention_swin_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I = ctypes.c_void_p, ctypes.c_int
_lib.swin_wattn_precompute.argtypes = [_I, _I, _I, _I, _P]
_lib.swin_wattn_fwd.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]
_lib.swin_wattn_fwd_f32.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]
_F = ctypes.c_float
_lib.swin_wattn_fwd_i8.argtypes = [_P, _F, _F, _F, _F, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]
_lib.swin_wattn_bwd.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]
for _n in ("swin_wattn_copy_index", "swin_wattn_copy_mask", "swin_wattn_copy_region"):
    getattr(_lib, _n).argtypes = [_I, _I, _I, _I, _P, _P]
_lib.swin_linear_pack_weight.argtypes = [_P, _P, _I, _I, _P]
_lib.swin_linear_fwd.argtypes = [_P, _P, _P, _P, _P, ctypes.c_longlong, _I, _I, _P]
_lib.swin_linear_i8_pack_weight.argtypes = [_P, _P, _I, _I, _P]
_lib.swin_linear_i8_fwd.argtypes = [_P, _F, _P, _P, _P, _P, _P, _P, ctypes.c_longlong, _I, _I, _P]
_lib.swin_ln_linear_pack_weight.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _P]
_lib.swin_ln_linear_fwd.argtypes = [_P, _P, _P, ctypes.c_float, _P, ctypes.c_longlong, _I, _I, _P]
_lib.swin_ln_qkv_wattn_fwd.argtypes = [_P, _P, _P, ctypes.c_float, _P, _P, _I, _I, _I, _I, _I, _I,
                                       _I, _P]
_lib.swin_wattn_release.argtypes = []
_lib.swin_wattn_status_string.argtypes = [_I]
_lib.swin_wattn_status_string.restype = ctypes.c_char_p
for _n in EXPORTS[:-1]:
    getattr(_lib, _n).restype = _I


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        if _torch is not None and _torch.cuda.is_available():
            return _torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream  # a torch.cuda.Stream


def swin_wattn_precompute(H: int, W: int, window: int, shift: int, stream=None) -> int:
    return _lib.swin_wattn_precompute(H, W, window, shift, _stream(stream))


def swin_wattn_fwd(qkv, rel_bias_table, out, B: int, H: int, W: int, heads: int, head_dim: int,
                   window: int, shift: int, stream=None) -> int:
    return _lib.swin_wattn_fwd(_addr(qkv), _addr(rel_bias_table), _addr(out), B, H, W, heads,
                               head_dim, window, shift, _stream(stream))


def swin_wattn_fwd_f32(qkv, rel_bias_table, out, B: int, H: int, W: int, heads: int,
                       head_dim: int, window: int, shift: int, stream=None) -> int:
    return _lib.swin_wattn_fwd_f32(_addr(qkv), _addr(rel_bias_table), _addr(out), B, H, W, heads,
                                   head_dim, window, shift, _stream(stream))


def swin_wattn_fwd_i8(qkv, scale_q: float, scale_k: float, scale_v: float, out_scale: float,
                      rel_bias_table, out, B: int, H: int, W: int, heads: int, head_dim: int,
                      window: int, shift: int, stream=None) -> int:
    return _lib.swin_wattn_fwd_i8(_addr(qkv), scale_q, scale_k, scale_v, out_scale,
                                  _addr(rel_bias_table), _addr(out), B, H, W, heads, head_dim,
                                  window, shift, _stream(stream))


def swin_wattn_bwd(qkv, rel_bias_table, dout, dqkv, dtable, B: int, H: int, W: int, heads: int,
                   head_dim: int, window: int, shift: int, stream=None) -> int:
    return _lib.swin_wattn_bwd(_addr(qkv), _addr(rel_bias_table), _addr(dout), _addr(dqkv),
                               _addr(dtable), B, H, W, heads, head_dim, window, shift,
                               _stream(stream))


def swin_wattn_copy_index(H: int, W: int, window: int, shift: int, dst, stream=None) -> int:
    return _lib.swin_wattn_copy_index(H, W, window, shift, _addr(dst), _stream(stream))


def swin_wattn_copy_mask(H: int, W: int, window: int, shift: int, dst, stream=None) -> int:
    return _lib.swin_wattn_copy_mask(H, W, window, shift, _addr(dst), _stream(stream))


def swin_wattn_copy_region(H: int, W: int, window: int, shift: int, dst, stream=None) -> int:
    return _lib.swin_wattn_copy_region(H, W, window, shift, _addr(dst), _stream(stream))


def swin_linear_pack_weight(weight, packed, N: int, K: int, stream=None) -> int:
    return _lib.swin_linear_pack_weight(_addr(weight), _addr(packed), N, K, _stream(stream))


def swin_linear_fwd(x, packed_weight, bias, residual, y, T: int, K: int, N: int,
                    stream=None) -> int:
    return _lib.swin_linear_fwd(_addr(x), _addr(packed_weight), _addr(bias), _addr(residual),
                                _addr(y), T, K, N, _stream(stream))


def swin_linear_i8_pack_weight(weight, packed, N: int, K: int, stream=None) -> int:
    return _lib.swin_linear_i8_pack_weight(_addr(weight), _addr(packed), N, K, _stream(stream))


def swin_linear_i8_fwd(x, x_scale: float, packed_weight, w_scale, bias, residual, out_scale, y,
                       T: int, K: int, N: int, stream=None) -> int:
    return _lib.swin_linear_i8_fwd(_addr(x), x_scale, _addr(packed_weight), _addr(w_scale),
                                   _addr(bias), _addr(residual), _addr(out_scale), _addr(y), T, K,
                                   N, _stream(stream))


def swin_ln_linear_pack_weight(weight, gamma, beta, bias, packed, consts, N: int, K: int,
                               stream=None) -> int:
    return _lib.swin_ln_linear_pack_weight(_addr(weight), _addr(gamma), _addr(beta), _addr(bias),
                                           _addr(packed), _addr(consts), N, K, _stream(stream))


def swin_ln_linear_fwd(x, packed_weight, consts, eps: float, y, T: int, K: int, N: int,
                       stream=None) -> int:
    return _lib.swin_ln_linear_fwd(_addr(x), _addr(packed_weight), _addr(consts), eps, _addr(y),
                                   T, K, N, _stream(stream))


def swin_ln_qkv_wattn_fwd(x, packed_qkv, consts, eps: float, rel_bias_table, out, B: int, H: int,
                          W: int, heads: int, head_dim: int, window: int, shift: int,
                          stream=None) -> int:
    return _lib.swin_ln_qkv_wattn_fwd(_addr(x), _addr(packed_qkv), _addr(consts), eps,
                                      _addr(rel_bias_table), _addr(out), B, H, W, heads, head_dim,
                                      window, shift, _stream(stream))


def swin_wattn_release() -> int:
    return _lib.swin_wattn_release()


def swin_wattn_status_string(status: int) -> str:
    return _lib.swin_wattn_status_string(status).decode()


def check(status: int, call: str = "") -> None:
    """Raises SwinAttnError for a non-zero status."""
    if status != SWIN_OK:
        raise SwinAttnError(status, call)


def library():
    """The loaded ctypes library (for symbol checks)."""
    return _lib
