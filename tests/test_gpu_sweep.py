"""Seeded sweep of random shapes: the bf16 forward, the INT8 forward (bf16
and int8 output), the backward, the linear layers (bf16 and INT8) and the
fused layer norm + QKV + attention against the fp64 oracle, at shapes drawn
from a fixed seed.

The draws cover windows 1-12, 1-16 heads, every shift, 1-3 images and
1-3 windows per axis (H != W included), so the launch plans of the
persistent kernels (head groups, grid order or XCD ranges, bias tables of
every head, of the workgroup's head group or restaged per unit, grid
tails) are exercised beyond the hand-picked cases.  Same bars as the other
parity tests.  Every case prints its shape before touching the GPU."""
import numpy as np
import pytest
import torch

import oracle
import shifted_window_attention_swin_amd as swa
import synth

pytestmark = pytest.mark.gpu


def _shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 13))
        s = int(rng.integers(0, M))
        nh = int(rng.integers(1, 17))
        B = int(rng.integers(1, 4))
        H, W = M * int(rng.integers(1, 4)), M * int(rng.integers(1, 4))
        out.append((B, H, W, nh, M, s))
    return out


def _dev():
    return torch.device("cuda:0")


def _check(got, ref, what):
    err = np.abs(got - ref)
    print(f"    {what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert np.isfinite(got).all(), what
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, what


@pytest.mark.parametrize("B,H,W,nh,M,s", _shapes(2024, 64))
def test_sweep_bf16_forward(B, H, W, nh, M, s):
    print(f"[case] sweep bf16 fwd B={B} H={H} W={W} nh={nh} M={M} s={s}", flush=True)
    qkv, table = synth.make_inputs(B, H, W, nh, 32, M, seed=4000 + B * 97 + H * 13 + nh, dtype="bf16")
    q = torch.from_numpy(qkv.view(np.int16)).view(torch.bfloat16).to(_dev())
    t = torch.from_numpy(table).to(_dev())
    out = torch.full((B, H, W, nh * 32), float("nan"), dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_wattn_fwd(q, t, out, B, H, W, nh, 32, M, s), "fwd")
    torch.cuda.synchronize()
    _check(out.float().cpu().numpy().astype(np.float64), oracle.swin_wattn_fwd(qkv, table, M, s), "bf16")


@pytest.mark.parametrize("B,H,W,nh,M,s", _shapes(2025, 48))
def test_sweep_i8_forward(B, H, W, nh, M, s):
    print(f"[case] sweep i8 fwd B={B} H={H} W={W} nh={nh} M={M} s={s}", flush=True)
    codes, scales, table = synth.make_i8_inputs(B, H, W, nh, 32, M, seed=5000 + B * 97 + H * 13 + nh)
    out = torch.full((B, H, W, nh * 32), float("nan"), dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_wattn_fwd_i8(torch.from_numpy(codes).to(_dev()), *(float(v) for v in scales), 0.0,
                                    torch.from_numpy(table).to(_dev()), out, B, H, W, nh, 32, M, s),
              "fwd_i8")
    torch.cuda.synchronize()
    _check(out.float().cpu().numpy().astype(np.float64),
           oracle.swin_wattn_fwd_i8(codes, scales, table, M, s), "i8")


@pytest.mark.parametrize("B,H,W,nh,M,s", _shapes(2026, 48))
def test_sweep_backward(B, H, W, nh, M, s):
    print(f"[case] sweep bwd B={B} H={H} W={W} nh={nh} M={M} s={s}", flush=True)
    qkv, table = synth.make_inputs(B, H, W, nh, 32, M, seed=6000 + B * 97 + H * 13 + nh, dtype="bf16")
    C = nh * 32
    dout = synth.bf16_bits(synth.normal(synth.stream_key(6000 + H, 7), B * H * W * C)).reshape(B, H, W, C)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(_dev())
    q, g, t = bf(qkv), bf(dout), torch.from_numpy(table).to(_dev())
    dq = torch.full_like(q, float("nan"))
    dt = torch.full_like(t, float("nan"))
    swa.check(swa.swin_wattn_bwd(q, t, g, dq, dt, B, H, W, nh, 32, M, s), "bwd")
    torch.cuda.synchronize()
    rq, rt = oracle.swin_wattn_bwd(qkv, table, dout, M, s)
    gq = dq.float().cpu().numpy().astype(np.float64)
    gt = dt.cpu().numpy().astype(np.float64)
    e, et = np.abs(gq - rq), np.abs(gt - rt)
    print(f"    dqkv max_abs={e.max():.3e} mean_abs={e.mean():.3e}; dtable max_err={et.max():.3e}", flush=True)
    assert np.isfinite(gq).all() and np.isfinite(gt).all()
    # the backward's bars (per gradient part, as in the backward parity tests)
    for part in range(3):
        ep, rp = e[:, :, :, part], rq[:, :, :, part]
        assert ep.max() <= 2.0 ** -6 * np.abs(rp).max() + 1e-6
        assert ep.mean() <= 2.0 ** -8 * np.abs(rp).mean() + 1e-7
    assert et.max() <= 1e-3 * np.abs(rt).max() + 1e-6


def _linear_shapes(seed, n, kmax):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 300)), 32 * int(rng.integers(1, kmax // 32 + 1)),
             32 * int(rng.integers(1, 40)), str(rng.choice(["plain", "res"]))) for _ in range(n)]


@pytest.mark.parametrize("T,K,N,mode", _linear_shapes(2027, 24, 384))
def test_sweep_linear(T, K, N, mode):
    print(f"[case] sweep linear T={T} K={K} N={N} {mode}", flush=True)
    x, w, b, r = synth.make_linear_inputs(T, K, N, 7000 + T + K, mode == "res")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(_dev())
    wd = bf(w)
    packed = torch.empty_like(wd)
    swa.check(swa.swin_linear_pack_weight(wd, packed, N, K), "pack")
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_linear_fwd(bf(x), packed, torch.from_numpy(b).to(_dev()),
                                  bf(r) if r is not None else None, y, T, K, N), "linear")
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    ref = oracle.linear(x, w, b, r)
    xf, wf = synth.bf16_to_f32(x).astype(np.float64), synth.bf16_to_f32(w).astype(np.float64)
    mag = np.abs(xf) @ np.abs(wf).T + np.abs(b)
    if r is not None:
        mag = mag + np.abs(synth.bf16_to_f32(r))
    assert (np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 2.0 ** -20 * mag).all()


@pytest.mark.parametrize("T,K,N,mode", [(t, k, n, m if m == "res" else "i8")
                                        for t, k, n, m in _linear_shapes(2028, 24, 768)])
def test_sweep_linear_i8(T, K, N, mode):
    print(f"[case] sweep linear i8 T={T} K={K} N={N} {mode}", flush=True)
    x, sx, w, sw, b, r, so = synth.make_linear_i8_inputs(T, K, N, 8000 + T + K, mode == "res",
                                                         mode == "i8")
    f32 = lambda a: None if a is None else torch.from_numpy(a).to(_dev())
    wd = torch.from_numpy(w).to(_dev())
    packed = torch.zeros(N * ((K + 63) // 64) * 64, dtype=torch.int8, device=_dev())
    swa.check(swa.swin_linear_i8_pack_weight(wd, packed, N, K), "pack_i8")
    if mode == "i8":
        y = torch.full((T, N), -128, dtype=torch.int8, device=_dev())
        rd = None
    else:
        y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=_dev())
        rd = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16).to(_dev())
    swa.check(swa.swin_linear_i8_fwd(torch.from_numpy(x).to(_dev()), float(sx), packed, f32(sw), f32(b),
                                     rd, f32(so), y, T, K, N), "linear_i8")
    torch.cuda.synchronize()
    _, ref, codes = oracle.linear_i8(x, sx, w, sw, b, residual=r, so=so)
    if mode == "i8":
        assert np.array_equal(y.cpu().numpy(), codes)
    else:
        got = y.float().cpu().numpy().astype(np.float64)
        mag = (np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T) * (float(sx) * sw) + np.abs(b) \
            + np.abs(synth.bf16_to_f32(r))
        assert (np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 2.0 ** -20 * mag).all()


@pytest.mark.parametrize("B,H,W,nh,M,s", _shapes(2030, 24))
def test_sweep_i8_forward_int8_out(B, H, W, nh, M, s):
    # int8 output codes (out_scale = max |o| / 127): each code within 1 of
    # the fp64 output's code (round half to even, clamped to +-127), nearly
    # all equal to it, never -128 (the fill value: a position never written)
    print(f"[case] sweep i8 fwd int8 out B={B} H={H} W={W} nh={nh} M={M} s={s}", flush=True)
    codes, scales, table = synth.make_i8_inputs(B, H, W, nh, 32, M, seed=5500 + B * 97 + H * 13 + nh)
    o64 = oracle.swin_wattn_fwd_i8(codes, scales, table, M, s)
    so = float(np.float32(np.abs(o64).max() / 127.0))
    out = torch.full((B, H, W, nh * 32), -128, dtype=torch.int8, device=_dev())
    swa.check(swa.swin_wattn_fwd_i8(torch.from_numpy(codes).to(_dev()), *(float(v) for v in scales), so,
                                    torch.from_numpy(table).to(_dev()), out, B, H, W, nh, 32, M, s),
              "fwd_i8 int8 out")
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    exact = np.clip(np.rint(o64 / so), -127, 127)
    d = np.abs(got - exact)
    print(f"    codes: max diff {d.max():.0f}, equal {np.mean(d == 0):.4f}", flush=True)
    assert got.min() >= -127 and d.max() <= 1 and np.mean(d == 0) >= 0.97


def _ln_attn_shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(5, 9))
        s = int(rng.integers(0, M))
        nh = int(rng.integers(1, 7))  # C = 32 .. 192
        B = int(rng.integers(1, 3))
        H, W = M * int(rng.integers(1, 4)), M * int(rng.integers(1, 4))
        out.append((B, H, W, nh, M, s))
    return out


@pytest.mark.parametrize("B,H,W,nh,M,s", _ln_attn_shapes(2029, 24))
def test_sweep_ln_attn(B, H, W, nh, M, s):
    print(f"[case] sweep ln_qkv_wattn B={B} H={H} W={W} nh={nh} M={M} s={s}", flush=True)
    x, g, be, w, b, t = synth.make_ln_attn_inputs(B, H, W, nh, M, seed=9000 + B * 97 + H * 13 + nh)
    C = nh * 32
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(_dev())
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(_dev())
    wd = bf(w)
    packed = torch.empty_like(wd)
    consts = torch.empty(2, 3 * C, dtype=torch.float32, device=_dev())
    swa.check(swa.swin_ln_linear_pack_weight(wd, f32(g), f32(be), f32(b), packed, consts, 3 * C, C),
              "pack")
    out = torch.full((B, H, W, C), float("nan"), dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_ln_qkv_wattn_fwd(bf(x), packed, consts, 1e-5, f32(t), out, B, H, W, nh, 32, M, s),
              "ln_qkv_wattn")
    torch.cuda.synchronize()
    qkv = oracle.linear(oracle.layernorm(x, g, be, 1e-5), w, b).reshape(B, H, W, 3, nh, 32)
    _check(out.float().cpu().numpy().astype(np.float64), oracle.swin_wattn_fwd(qkv, t, M, s), "ln_attn")
