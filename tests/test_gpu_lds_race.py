"""LDS race check: a kernel that reads LDS it has not written (or reads it
before another wave's write has landed) gives results that depend on what
the LDS held before it ran.  Each kernel here runs twice, each time right
after a scrub that fills the LDS of every compute unit with different
seeded words (tests/support/lds_scrub.hip, same stream); both results must
be bit-identical and match the fp64 oracle.  The bias-table gradient of the
backward is a sum of fp32 atomics whose order varies between runs, so it is
compared to the oracle only.  Every case prints its name before touching
the GPU."""
import numpy as np
import pytest
import torch

import oracle
import shifted_window_attention_swin_amd as swa
import synth
from tests.support import lds_scrub

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _dev():
    return torch.device("cuda:0")


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(_dev())


def _twice(run):
    """run() queues the kernel and returns its output tensors; returns the
    results of two runs, each after a scrub with its own seed."""
    outs = []
    for seed in (0x5eed0001, 0xc0ffee02):
        torch.cuda.synchronize()
        lds_scrub(seed, torch.cuda.current_stream().cuda_stream)
        res = run()
        torch.cuda.synchronize()
        outs.append([t.clone() for t in res])
    return outs


@pytest.mark.parametrize("B,H,W,nh,M,s,dtype", [
    (4, 56, 56, 6, 7, 3, "bf16"),    # persistent, two-head units, grid order
    (2, 96, 96, 6, 12, 6, "bf16"),   # persistent, window 12, one head's bias, XCD ranges
    (8, 14, 14, 12, 7, 3, "bf16"),   # small launch in XCD ranges
    (2, 14, 14, 3, 7, 3, "bf16"),    # three-head units (operands held)
    (1, 14, 14, 64, 7, 3, "bf16"),   # 64 heads: one head group's tables, staged per unit
    (1, 12, 12, 48, 12, 0, "bf16"),  # window 12, 48 heads: tables staged per unit
    (2, 28, 14, 3, 7, 3, "f32"),     # fp32 kernel
])
def test_forward_independent_of_stale_lds(B, H, W, nh, M, s, dtype):
    _say(f"lds race fwd B={B} H={H} W={W} nh={nh} M={M} s={s} {dtype}")
    qkv, table = synth.make_inputs(B, H, W, nh, 32, M, seed=900 + M + nh, dtype=dtype)
    if dtype == "bf16":
        q, fn, tdt = _bf16_dev(qkv), swa.swin_wattn_fwd, torch.bfloat16
    else:
        q, fn, tdt = torch.from_numpy(qkv).to(_dev()), swa.swin_wattn_fwd_f32, torch.float32
    t = torch.from_numpy(table).to(_dev())
    out = torch.empty(B, H, W, nh * 32, dtype=tdt, device=_dev())

    def run():
        out.fill_(float("nan"))
        swa.check(fn(q, t, out, B, H, W, nh, 32, M, s), "fwd")
        return [out]

    (a,), (b,) = _twice(run)
    assert torch.equal(a, b), "forward output depends on the LDS contents before the launch"
    got = a.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - oracle.swin_wattn_fwd(qkv, table, M, s))
    print(f"    max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert np.isfinite(got).all()
    if dtype == "bf16":
        assert err.max() <= 2e-2 and err.mean() <= 2e-3
    else:
        assert err.max() <= 1e-4


@pytest.mark.parametrize("B,H,W,nh,M,s", [
    (2, 56, 56, 6, 7, 3),    # head pairs, whole-line stores through LDS
    (2, 14, 14, 3, 7, 3),    # one head per workgroup
    (1, 96, 96, 6, 12, 6),   # window 12
    (2, 24, 36, 3, 12, 5),
])
def test_backward_independent_of_stale_lds(B, H, W, nh, M, s):
    _say(f"lds race bwd B={B} H={H} W={W} nh={nh} M={M} s={s}")
    qkv, table = synth.make_inputs(B, H, W, nh, 32, M, seed=950 + M + nh, table_std=0.3)
    C = nh * 32
    dout = synth.bf16_bits(synth.normal(synth.stream_key(960 + M, 7), B * H * W * C, 1.0)).reshape(B, H, W, C)
    q, g, t = _bf16_dev(qkv), _bf16_dev(dout), torch.from_numpy(table).to(_dev())
    dq = torch.empty_like(q)
    dt = torch.empty_like(t)

    def run():
        dq.fill_(float("nan"))
        swa.check(swa.swin_wattn_bwd(q, t, g, dq, dt, B, H, W, nh, 32, M, s), "bwd")
        return [dq, dt]

    (a, ta), (b, tb) = _twice(run)
    assert torch.equal(a, b), "dqkv depends on the LDS contents before the launch"
    rq, rt = oracle.swin_wattn_bwd(qkv, table, dout, M, s)
    got = a.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    for i, comp in enumerate("qkv"):
        e = np.abs(got[:, :, :, i] - rq[:, :, :, i])
        ref = np.abs(rq[:, :, :, i])
        print(f"    d{comp}: max_abs={e.max():.3e} mean_abs={e.mean():.3e}", flush=True)
        assert e.max() <= 2.0**-6 * ref.max() + 1e-6 and e.mean() <= 2.0**-8 * ref.mean() + 1e-7
    for dt_run in (ta, tb):
        et = np.abs(dt_run.cpu().numpy().astype(np.float64) - rt).max()
        assert et <= 1e-3 * np.abs(rt).max() + 1e-6


@pytest.mark.parametrize("layernorm", [False, True])
def test_linear_independent_of_stale_lds(layernorm):
    T, K, N = 3 * 1024 + 40, 192, 576
    _say(f"lds race linear T={T} K={K} N={N} layernorm={layernorm}")
    rng_x = synth.normal(synth.stream_key(971, 1), T * K, 1.0)
    x_bits = synth.bf16_bits(2.0 * rng_x + 0.5).reshape(T, K)
    w_bits = synth.bf16_bits(synth.normal(synth.stream_key(971, 2), N * K, 0.02)).reshape(N, K)
    bias = synth.normal(synth.stream_key(971, 3), N, 0.02).astype(np.float32)
    x, w, b = _bf16_dev(x_bits), _bf16_dev(w_bits), torch.from_numpy(bias).to(_dev())
    packed = torch.empty_like(w)
    y = torch.empty(T, N, dtype=torch.bfloat16, device=_dev())
    if layernorm:
        gamma = (1.0 + synth.normal(synth.stream_key(971, 4), K, 0.1)).astype(np.float32)
        beta = synth.normal(synth.stream_key(971, 5), K, 0.1).astype(np.float32)
        consts = torch.empty(2, N, dtype=torch.float32, device=_dev())
        swa.check(swa.swin_ln_linear_pack_weight(w, torch.from_numpy(gamma).to(_dev()),
                                                 torch.from_numpy(beta).to(_dev()), b, packed,
                                                 consts, N, K), "pack")
    else:
        swa.check(swa.swin_linear_pack_weight(w, packed, N, K), "pack")

    def run():
        y.fill_(float("nan"))
        if layernorm:
            swa.check(swa.swin_ln_linear_fwd(x, packed, consts, 1e-5, y, T, K, N), "ln_linear")
        else:
            swa.check(swa.swin_linear_fwd(x, packed, b, None, y, T, K, N), "linear")
        return [y]

    (a,), (c,) = _twice(run)
    assert torch.equal(a, c), "linear output depends on the LDS contents before the launch"
    got = a.float().cpu().numpy().astype(np.float64)
    xr = synth.bf16_to_f32(x_bits).astype(np.float64)
    if layernorm:
        xr = oracle.layernorm(x_bits, gamma, beta)
    ref = oracle.linear(xr if layernorm else x_bits, w_bits, bias)
    mag = np.abs(xr) @ np.abs(synth.bf16_to_f32(w_bits).astype(np.float64)).T + np.abs(bias)
    err = np.abs(got - ref)
    lim = 2.0**-7 * np.abs(ref) + 2.0**-7 * mag
    print(f"    worst err/bound={float((err / lim).max()):.3f}", flush=True)
    assert np.isfinite(got).all() and (err <= lim).all()


def test_ln_attn_independent_of_stale_lds():
    B, H, W, nh, M, s = 2, 28, 28, 6, 7, 3
    _say(f"lds race ln_qkv_wattn B={B} H={H} W={W} nh={nh} M={M} s={s}")
    x, g, be, w, b, t = synth.make_ln_attn_inputs(B, H, W, nh, M, seed=977)
    C = 32 * nh
    wd = _bf16_dev(w)
    packed = torch.empty_like(wd)
    consts = torch.empty(2, 3 * C, dtype=torch.float32, device=_dev())
    swa.check(swa.swin_ln_linear_pack_weight(wd, torch.from_numpy(g).to(_dev()),
                                             torch.from_numpy(be).to(_dev()),
                                             torch.from_numpy(b).to(_dev()), packed, consts,
                                             3 * C, C), "pack")
    xd, td = _bf16_dev(x), torch.from_numpy(t).to(_dev())
    out = torch.empty(B, H, W, C, dtype=torch.bfloat16, device=_dev())

    def run():
        out.fill_(float("nan"))
        swa.check(swa.swin_ln_qkv_wattn_fwd(xd, packed, consts, 1e-5, td, out, B, H, W, nh, 32, M,
                                            s), "ln_qkv_wattn")
        return [out]

    (a,), (c,) = _twice(run)
    assert torch.equal(a, c), "fused output depends on the LDS contents before the launch"
    xn = oracle.layernorm(x, g, be)
    ref = oracle.swin_wattn_fwd(oracle.linear(xn, w, b).reshape(B, H, W, 3, nh, 32), t, M, s)
    err = np.abs(a.float().cpu().numpy().astype(np.float64) - ref)
    print(f"    max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3



@pytest.mark.parametrize("B,H,W,nh,M,s", [
    (4, 56, 56, 6, 7, 3),    # two-head units
    (2, 96, 96, 6, 12, 6),   # window 12, one head's bias
])
def test_forward_i8_independent_of_stale_lds(B, H, W, nh, M, s):
    _say(f"lds race fwd i8 B={B} H={H} W={W} nh={nh} M={M} s={s}")
    codes, scales, table = synth.make_i8_inputs(B, H, W, nh, 32, M, seed=950 + M + nh)
    q = torch.from_numpy(codes).to(_dev())
    t = torch.from_numpy(table).to(_dev())
    out = torch.empty(B, H, W, nh * 32, dtype=torch.bfloat16, device=_dev())

    def run():
        out.fill_(float("nan"))
        swa.check(swa.swin_wattn_fwd_i8(q, *(float(v) for v in scales), 0.0, t, out, B, H, W, nh, 32,
                                        M, s), "fwd_i8")
        return [out]

    (a,), (c,) = _twice(run)
    assert torch.equal(a, c), "INT8 forward output depends on the LDS contents before the launch"
    err = np.abs(a.float().cpu().numpy().astype(np.float64)
                 - oracle.swin_wattn_fwd_i8(codes, scales, table, M, s))
    print(f"    max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


@pytest.mark.parametrize("K,N,mode", [(192, 576, "i8"), (96, 288, "i8"), (192, 192, "res")])
def test_linear_i8_independent_of_stale_lds(K, N, mode):
    T = 3 * 1024 + 40
    _say(f"lds race linear i8 T={T} K={K} N={N} mode={mode}")
    x, sx, w, sw, bias, res, so = synth.make_linear_i8_inputs(T, K, N, 980 + K, mode == "res",
                                                              mode == "i8")
    f32 = lambda a: None if a is None else torch.from_numpy(a).to(_dev())
    xd, wd, swd, bd, sod = torch.from_numpy(x).to(_dev()), torch.from_numpy(w).to(_dev()), f32(sw), \
        f32(bias), f32(so)
    rd = _bf16_dev(res) if res is not None else None
    packed = torch.zeros(N * ((K + 63) // 64) * 64, dtype=torch.int8, device=_dev())
    swa.check(swa.swin_linear_i8_pack_weight(wd, packed, N, K), "pack_i8")
    y = torch.empty(T, N, dtype=torch.int8 if mode == "i8" else torch.bfloat16, device=_dev())

    def run():
        y.fill_(-128 if mode == "i8" else float("nan"))
        swa.check(swa.swin_linear_i8_fwd(xd, float(sx), packed, swd, bd, rd, sod, y, T, K, N),
                  "linear_i8")
        return [y]

    (a,), (c,) = _twice(run)
    assert torch.equal(a, c), "INT8 linear output depends on the LDS contents before the launch"
    _, ref, codes = oracle.linear_i8(x, sx, w, sw, bias, residual=res, so=so)
    if mode == "i8":
        assert np.array_equal(a.cpu().numpy(), codes)
    else:
        got = a.float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        assert (err <= 2.0**-7 * np.abs(ref) + 2.0**-7 * (np.abs(ref) + 1.0)).all()
