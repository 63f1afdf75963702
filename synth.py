"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no step of the attention method: it only draws numbers.
Both sides of every parity check read the very same arrays produced here.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) used in counter form -- draw k of a stream is
the SplitMix64 output for state ``key + (k+1) * golden`` -- so any slice of a
stream can be produced independently.  Uniforms take the top 53 bits; normals
come from the Box-Muller transform (Box and Muller, 1958), one pair of normals
per pair of uniforms, computed in float64, scaled by the std, then rounded to
float32 (and, for bfloat16 tensors, rounded again to nearest-even bfloat16).

Workload shapes are Swin stage shapes: qkv ``[B, H, W, 3, heads, head_dim]``
~ N(0, 1) and a relative position bias table ``[(2M-1)^2, heads]`` ~ N(0, 0.02).
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> int:
    """Independent 64-bit key for sub-stream ``stream`` of ``seed``."""
    z = np.array([(seed * 0x100000001B3 + stream) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    return int(_mix(z + _GOLDEN)[0])


def splitmix64(key: int, start: int, n: int) -> np.ndarray:
    """Draws ``start .. start+n-1`` of the SplitMix64 stream with state ``key``."""
    k = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(np.uint64(key) + k * _GOLDEN)


def uniform53(key: int, start: int, n: int) -> np.ndarray:
    """Uniform doubles in [0, 1) from the top 53 bits of each draw."""
    return (splitmix64(key, start, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(key: int, n: int, std: float = 1.0) -> np.ndarray:
    """``n`` normal float32 values; normal 2p and 2p+1 use draws 2p and 2p+1."""
    out = np.empty(n, dtype=np.float32)
    pairs = (n + 1) // 2
    for p0 in range(0, pairs, _CHUNK):
        p1 = min(pairs, p0 + _CHUNK)
        u = uniform53(key, 2 * p0, 2 * (p1 - p0))
        u1 = 1.0 - u[0::2]  # (0, 1]: keeps the log finite
        u2 = u[1::2]
        r = np.sqrt(-2.0 * np.log(u1))
        z = np.empty(2 * (p1 - p0), dtype=np.float64)
        z[0::2] = r * np.cos(2.0 * np.pi * u2)
        z[1::2] = r * np.sin(2.0 * np.pi * u2)
        lo, hi = 2 * p0, min(n, 2 * p1)
        out[lo:hi] = (z[: hi - lo] * std).astype(np.float32)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; returns the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 patterns."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Workloads: Swin stage shapes.  Each carries its own seed.

WORKLOADS = {
    "tiny-f32": dict(B=1, H=14, W=14, heads=2, head_dim=32, window=7, shifts=(3,), dtype="f32",
                     seed=1001, desc="tiny fp32 check, 14x14 tokens, window 7, shift 3"),
    "swin-t-s1": dict(B=32, H=56, W=56, heads=3, head_dim=32, window=7, shifts=(3,), dtype="bf16",
                      seed=1002, desc="Swin-T stage 1, B=32, 56x56, C=96"),
    "swin-t-s3": dict(B=64, H=14, W=14, heads=12, head_dim=32, window=7, shifts=(0, 3), dtype="bf16",
                      seed=1003, desc="Swin-T stage 3, B=64, 14x14, C=384, shift 0 and 3"),
    "swin-l-s1": dict(B=64, H=56, W=56, heads=6, head_dim=32, window=7, shifts=(3,), dtype="bf16",
                      seed=1004, desc="Swin-L stage 1, B=64, 56x56, C=192"),
    "swin-l-384": dict(B=16, H=96, W=96, heads=6, head_dim=32, window=12, shifts=(6,), dtype="bf16",
                       seed=1005, desc="Swin-L at 384px, B=16, 96x96, C=192, window 12"),
}


def make_inputs(B: int, H: int, W: int, heads: int, head_dim: int, window: int, seed: int,
                dtype: str = "bf16", qkv_std: float = 1.0, table_std: float = 0.02):
    """Returns ``(qkv, table)`` as numpy arrays.

    ``qkv`` is ``[B, H, W, 3, heads, head_dim]``: float32 values for ``dtype='f32'``,
    uint16 bfloat16 patterns for ``dtype='bf16'``.  ``table`` is float32
    ``[(2*window-1)**2, heads]``.
    """
    n = B * H * W * 3 * heads * head_dim
    q = normal(stream_key(seed, 0), n, qkv_std).reshape(B, H, W, 3, heads, head_dim)
    T = (2 * window - 1) ** 2
    table = normal(stream_key(seed, 1), T * heads, table_std).reshape(T, heads)
    if dtype == "bf16":
        q = bf16_bits(q)
    elif dtype != "f32":
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    return q, table


def workload_inputs(name: str, batch: int | None = None):
    """Inputs of a named workload (optionally with a smaller batch)."""
    w = WORKLOADS[name]
    B = w["B"] if batch is None else batch
    return make_inputs(B, w["H"], w["W"], w["heads"], w["head_dim"], w["window"], w["seed"],
                       w["dtype"])


# ---------------------------------------------------------------------------
# Linear-layer workloads on either side of the attention, at Swin stage
# shapes: the QKV projection (K = C, N = 3C, with bias) and the output
# projection (K = N = C, with bias and residual).  tokens = B * H * W.

LINEAR_WORKLOADS = {
    "qkv-t-s1": dict(tokens=32 * 56 * 56, K=96, N=288, residual=False, seed=2001,
                     desc="Swin-T stage 1 QKV projection, B=32, 56x56, C=96"),
    "qkv-t-s3": dict(tokens=64 * 14 * 14, K=384, N=1152, residual=False, seed=2002,
                     desc="Swin-T stage 3 QKV projection, B=64, 14x14, C=384"),
    "qkv-l-s1": dict(tokens=64 * 56 * 56, K=192, N=576, residual=False, seed=2003,
                     desc="Swin-L stage 1 QKV projection, B=64, 56x56, C=192"),
    "proj-l-s1": dict(tokens=64 * 56 * 56, K=192, N=192, residual=True, seed=2004,
                      desc="Swin-L stage 1 output projection + residual, B=64, 56x56, C=192"),
    "proj-t-s3": dict(tokens=64 * 14 * 14, K=384, N=384, residual=True, seed=2005,
                      desc="Swin-T stage 3 output projection + residual, B=64, 14x14, C=384"),
}


def make_linear_inputs(T: int, K: int, N: int, seed: int, residual: bool,
                       x_std: float = 1.0, w_std: float = 0.02, bias_std: float = 0.02):
    """Returns ``(x, w, bias, res)``: ``x [T, K]`` and ``w [N, K]`` as bfloat16
    patterns, ``bias [N]`` float32, ``res [T, N]`` bfloat16 patterns or None.
    A smaller T gives a prefix of the tokens of a larger one."""
    x = bf16_bits(normal(stream_key(seed, 0), T * K, x_std)).reshape(T, K)
    w = bf16_bits(normal(stream_key(seed, 1), N * K, w_std)).reshape(N, K)
    bias = normal(stream_key(seed, 2), N, bias_std)
    res = bf16_bits(normal(stream_key(seed, 3), T * N, 1.0)).reshape(T, N) if residual else None
    return x, w, bias, res


def linear_inputs(name: str, tokens: int | None = None):
    """Inputs of a named linear workload (optionally its first `tokens` tokens)."""
    w = LINEAR_WORKLOADS[name]
    T = w["tokens"] if tokens is None else tokens
    return make_linear_inputs(T, w["K"], w["N"], w["seed"], w["residual"])


# ---------------------------------------------------------------------------
# Layer norm + QKV projection workloads: x with a nonzero mean and spread
# (2 z + 0.5), gamma = 1 + 0.1 z, beta = 0.1 z, W and bias as above.

LN_LINEAR_WORKLOADS = {
    "lnqkv-t-s1": dict(tokens=32 * 56 * 56, K=96, N=288, seed=3001,
                       desc="Swin-T stage 1 layer norm + QKV projection, B=32, 56x56, C=96"),
    "lnqkv-t-s3": dict(tokens=64 * 14 * 14, K=384, N=1152, seed=3002,
                       desc="Swin-T stage 3 layer norm + QKV projection, B=64, 14x14, C=384"),
    "lnqkv-l-s1": dict(tokens=64 * 56 * 56, K=192, N=576, seed=3003,
                       desc="Swin-L stage 1 layer norm + QKV projection, B=64, 56x56, C=192"),
}


def make_ln_linear_inputs(T: int, K: int, N: int, seed: int):
    """Returns ``(x, gamma, beta, w, bias)``: ``x [T, K]`` and ``w [N, K]`` as
    bfloat16 patterns, ``gamma, beta [K]`` and ``bias [N]`` float32."""
    x = bf16_bits(normal(stream_key(seed, 0), T * K, 2.0) + np.float32(0.5)).reshape(T, K)
    gamma = normal(stream_key(seed, 1), K, 0.1) + np.float32(1.0)
    beta = normal(stream_key(seed, 2), K, 0.1)
    w = bf16_bits(normal(stream_key(seed, 3), N * K, 0.02)).reshape(N, K)
    bias = normal(stream_key(seed, 4), N, 0.02)
    return x, gamma, beta, w, bias


def ln_linear_inputs(name: str, tokens: int | None = None):
    """Inputs of a named layer norm + linear workload (optionally its first tokens)."""
    w = LN_LINEAR_WORKLOADS[name]
    T = w["tokens"] if tokens is None else tokens
    return make_ln_linear_inputs(T, w["K"], w["N"], w["seed"])


# ---------------------------------------------------------------------------
# Layer norm + QKV projection + window attention workloads (the attention
# half of a Swin block, before its output projection): x, gamma, beta, the
# QKV weight and bias of a layer norm + QKV workload (x as [B, H, W, C]),
# and the bias table of an attention workload of the same stage.

LN_ATTN_WORKLOADS = {
    "lnattn-l-s1": dict(ln="lnqkv-l-s1", attn="swin-l-s1",
                        desc="Swin-L stage 1 layer norm + QKV + window attention, B=64, 56x56, C=192"),
    "lnattn-t-s1": dict(ln="lnqkv-t-s1", attn="swin-t-s1",
                        desc="Swin-T stage 1 layer norm + QKV + window attention, B=32, 56x56, C=96"),
}


def attention_table(seed: int, heads: int, window: int, table_std: float = 0.02) -> np.ndarray:
    """The bias table ``make_inputs`` draws for ``seed`` (sub-stream 1),
    without drawing qkv."""
    T = (2 * window - 1) ** 2
    return normal(stream_key(seed, 1), T * heads, table_std).reshape(T, heads)


def make_ln_attn_inputs(B: int, H: int, W: int, heads: int, window: int, seed: int):
    """Returns ``(x [B,H,W,C], gamma, beta, w [3C, C], bias [3C], table)`` with
    C = 32 heads: the layer norm + QKV recipe for B*H*W tokens and the
    attention table of the same seed."""
    C = 32 * heads
    x, gamma, beta, w, bias = make_ln_linear_inputs(B * H * W, C, 3 * C, seed)
    return x.reshape(B, H, W, C), gamma, beta, w, bias, attention_table(seed, heads, window)


def ln_attn_inputs(name: str, batch: int | None = None):
    """Inputs of a named layer norm + attention workload (optionally its
    first images): those of its layer norm + QKV workload and the table of
    its attention workload."""
    spec = LN_ATTN_WORKLOADS[name]
    a = WORKLOADS[spec["attn"]]
    B = a["B"] if batch is None else batch
    T = B * a["H"] * a["W"]
    x, gamma, beta, w, bias = ln_linear_inputs(spec["ln"], tokens=T)
    C = a["heads"] * a["head_dim"]
    table = attention_table(a["seed"], a["heads"], a["window"])
    return x.reshape(B, a["H"], a["W"], C), gamma, beta, w, bias, table



# ---------------------------------------------------------------------------
# INT8 workloads: integer codes drawn from a normal of std 32, rounded to the
# nearest integer and clipped to [-127, 127] (about 1 draw in 10^4 sits at
# an end), and one float32 scale per tensor or channel.  The codes and the
# scales are the inputs; nothing here quantizes a floating-point tensor.

def int8_codes(key: int, n: int, std: float = 32.0) -> np.ndarray:
    """``n`` int8 codes: rounded normal draws of ``std``, clipped to +-127."""
    return np.clip(np.rint(normal(key, n, std)), -127, 127).astype(np.int8)


# INT8 attention: q, k, v codes with one scale each (dequantized std about 1),
# at the shapes of the bf16 attention workloads (same seeds, same bias table)
I8_ATTN_SCALES = (0.031, 0.029, 0.033)
I8_WORKLOADS = {
    "swin-l-s1-i8": dict(attn="swin-l-s1", desc="Swin-L stage 1, B=64, 56x56, C=192, INT8 q/k/v"),
    "swin-t-s1-i8": dict(attn="swin-t-s1", desc="Swin-T stage 1, B=32, 56x56, C=96, INT8 q/k/v"),
    "swin-t-s3-i8": dict(attn="swin-t-s3", desc="Swin-T stage 3, B=64, 14x14, C=384, INT8 q/k/v"),
    "swin-l-384-i8": dict(attn="swin-l-384", desc="Swin-L at 384px, B=16, 96x96, C=192, window 12, "
                                                   "INT8 q/k/v"),
}


def make_i8_inputs(B: int, H: int, W: int, heads: int, head_dim: int, window: int, seed: int,
                   scales=I8_ATTN_SCALES):
    """Returns ``(codes [B,H,W,3,heads,head_dim] int8, scales [3] float32,
    table [(2*window-1)**2, heads] float32)``."""
    n = B * H * W * 3 * heads * head_dim
    codes = int8_codes(stream_key(seed, 10), n).reshape(B, H, W, 3, heads, head_dim)
    return codes, np.array(scales, dtype=np.float32), attention_table(seed, heads, window)


def i8_inputs(name: str, batch: int | None = None):
    """Inputs of a named INT8 attention workload (optionally its first images)."""
    a = WORKLOADS[I8_WORKLOADS[name]["attn"]]
    B = a["B"] if batch is None else batch
    return make_i8_inputs(B, a["H"], a["W"], a["heads"], a["head_dim"], a["window"], a["seed"])


# INT8 linear layers: x codes (scale 1/32, so x is about N(0, 1)), weight
# codes with per-row scales (W about N(0, 0.02)), bias ~ N(0, 0.02).  The
# QKV projections write INT8 with one output scale per part (query, key,
# value: about 4 output spreads over 127, the scales swin_wattn_fwd_i8
# reads); the output projection writes bf16 and adds a bf16 residual.
LINEAR_I8_WORKLOADS = {
    "qkv-l-s1-i8": dict(tokens=64 * 56 * 56, K=192, N=576, residual=False, out_i8=True, seed=2101,
                        desc="Swin-L stage 1 QKV projection, B=64, 56x56, C=192, INT8 in and out"),
    "qkv-t-s1-i8": dict(tokens=32 * 56 * 56, K=96, N=288, residual=False, out_i8=True, seed=2102,
                        desc="Swin-T stage 1 QKV projection, B=32, 56x56, C=96, INT8 in and out"),
    "proj-l-s1-i8": dict(tokens=64 * 56 * 56, K=192, N=192, residual=True, out_i8=False, seed=2103,
                         desc="Swin-L stage 1 output projection + residual, B=64, 56x56, C=192, "
                              "INT8 in, bf16 out"),
}
I8_QKV_PART_SCALES = (1.0, 0.9, 1.1)  # relative output scales of query, key, value


def make_linear_i8_inputs(T: int, K: int, N: int, seed: int, residual: bool, out_i8: bool):
    """Returns ``(x [T,K] int8, x_scale float32, w [N,K] int8, w_scale [N]
    float32, bias [N] float32, res [T,N] bf16 patterns or None, out_scale [N]
    float32 or None)``.  A smaller T gives a prefix of the tokens of a larger one."""
    x = int8_codes(stream_key(seed, 0), T * K).reshape(T, K)
    w = int8_codes(stream_key(seed, 1), N * K).reshape(N, K)
    x_scale = np.float32(1.0 / 32.0)
    spread = np.clip(normal(stream_key(seed, 2), N, 0.1) + np.float32(1.0), 0.5, 1.5)
    w_scale = (spread * np.float32(0.02 / 32.0)).astype(np.float32)
    bias = normal(stream_key(seed, 3), N, 0.02)
    res = bf16_bits(normal(stream_key(seed, 4), T * N, 1.0)).reshape(T, N) if residual else None
    out_scale = None
    if out_i8:
        base = np.float32(4.0 * 0.02 * np.sqrt(K) / 127.0)
        part = np.repeat(np.array(I8_QKV_PART_SCALES, dtype=np.float32), N // 3) if N % 3 == 0 else \
            np.ones(N, dtype=np.float32)
        out_scale = (base * part).astype(np.float32)
    return x, x_scale, w, w_scale, bias, res, out_scale


def linear_i8_inputs(name: str, tokens: int | None = None):
    """Inputs of a named INT8 linear workload (optionally its first tokens)."""
    w = LINEAR_I8_WORKLOADS[name]
    T = w["tokens"] if tokens is None else tokens
    return make_linear_i8_inputs(T, w["K"], w["N"], w["seed"], w["residual"], w["out_i8"])
