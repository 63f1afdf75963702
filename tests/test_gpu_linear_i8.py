"""GPU parity of the INT8 linear layer (swin_linear_i8_fwd) against the fp64
oracle, through the C ABI.

INT8 output: the codes are decided in fp32 by the same operations on both
sides (the integer sum exact, one fused multiply-add, round half to even,
clamp), so they must agree bit for bit.  bf16 output, per element:
|gpu - oracle| <= 2^-7 |oracle| + 2^-20 (sum_c |x_c w_c| sx sw_j + |bias| +
|residual|): the integer sum is exact (|sum| < 2^24 at K <= 768), the fp32
scaling and additions add a few 2^-24 relative errors, and the bf16 rounding
2^-8 relative; the bound takes twice that.  Inputs are the seeded workloads
of synth.py.  Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import shifted_window_attention_swin_amd as swa
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _dev():
    return torch.device("cuda:0")


def _i8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(_dev())


def _f32_dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(_dev())


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(_dev())


def _pack(w):
    N, K = w.shape
    wd = _i8_dev(w)
    packed = torch.zeros(N * ((K + 63) // 64) * 64, dtype=torch.int8, device=_dev())
    swa.check(swa.swin_linear_i8_pack_weight(wd, packed, N, K), "pack_i8")
    return packed


def _run(x, sx, w, sw, bias, res_bits=None, so=None, inplace=False):
    """One swin_linear_i8_fwd; returns the output on the host (int8 codes,
    or float64 of the bf16 values)."""
    T, K = x.shape
    N = w.shape[0]
    packed = _pack(w)
    xd, swd, bd, sod = _i8_dev(x), _f32_dev(sw), _f32_dev(bias), _f32_dev(so)
    if so is not None:
        # -128 is no code (codes are clamped to +-127): any left is a position never written
        y = torch.full((T, N), -128, dtype=torch.int8, device=_dev())
        r = None
    elif inplace:
        y = _bf16_dev(res_bits)
        r = y
    else:
        r = _bf16_dev(res_bits) if res_bits is not None else None
        y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_linear_i8_fwd(xd, float(sx), packed, swd, bd, r, sod, y, T, K, N), "linear_i8")
    torch.cuda.synchronize()
    if so is not None:
        assert bool((y != -128).all())
        return y.cpu().numpy()
    assert bool(torch.isfinite(y).all())
    return y.float().cpu().numpy().astype(np.float64)


def _check_bf16(got, ref, x, sx, w, sw, bias, res_bits, what):
    mag = (np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T) * (float(sx) * sw.astype(np.float64))
    if bias is not None:
        mag = mag + np.abs(bias.astype(np.float64))
    if res_bits is not None:
        mag = mag + np.abs(synth.bf16_to_f32(res_bits).astype(np.float64))
    err = np.abs(got - ref)
    bound = 2.0 ** -7 * np.abs(ref) + 2.0 ** -20 * mag
    print(f"    {what}: max_abs={err.max():.3e} worst err/bound={np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound), what


def _check_codes(got, ref, what):
    diff = int(np.count_nonzero(got != ref))
    print(f"    {what}: {diff} of {ref.size} codes differ; saturated {np.mean(np.abs(ref) == 127):.4f}",
          flush=True)
    assert diff == 0, what


@pytest.mark.parametrize("T,K,N,mode", [
    (1, 64, 32, "bf16"),
    (33, 96, 288, "i8"),        # K = 96: a last half k-step
    (100, 192, 576, "i8"),      # Swin-L QKV shape, ragged row blocks
    (77, 192, 192, "res"),
    (64, 384, 1152, "i8"),
    (45, 768, 256, "bf16"),     # the largest K
    (31, 32, 64, "i8"),         # one half k-step only
    (65, 160, 96, "res"),       # 2.5 k-steps, N / 32 = 3 column blocks (2-wave groups)
    (40, 128, 128, "inplace"),  # residual added in place
    (0, 192, 576, "i8"),        # empty
])
def test_linear_i8_shapes(T, K, N, mode):
    _say(f"linear_i8 T={T} K={K} N={N} mode={mode}")
    x, sx, w, sw, bias, res, so = synth.make_linear_i8_inputs(T, K, N, 700 + K + N,
                                                              mode in ("res", "inplace"), mode == "i8")
    if T == 0:
        packed = _pack(w)
        y = torch.full((1, N), 5, dtype=torch.int8, device=_dev())
        assert swa.swin_linear_i8_fwd(1 << 20, float(sx), packed, _f32_dev(sw), _f32_dev(bias), None,
                                      _f32_dev(so), y, 0, K, N) == swa.SWIN_OK
        torch.cuda.synchronize()
        assert bool((y == 5).all())
        return
    got = _run(x, sx, w, sw, bias, res, so, inplace=mode == "inplace")
    acc, ref, codes = oracle.linear_i8(x, sx, w, sw, bias, residual=res, so=so)
    if mode == "i8":
        _check_codes(got, codes, "codes")
    else:
        _check_bf16(got, ref, x, sx, w, sw, bias, res, "bf16 out")


@pytest.mark.parametrize("name", ["qkv-l-s1-i8", "qkv-t-s1-i8", "proj-l-s1-i8"])
def test_linear_i8_workloads_full(name):
    # the whole workload (the benchmark's launch); every output compared
    spec = synth.LINEAR_I8_WORKLOADS[name]
    _say(f"linear_i8 {name} full T={spec['tokens']}")
    x, sx, w, sw, bias, res, so = synth.linear_i8_inputs(name)
    got = _run(x, sx, w, sw, bias, res, so)
    if so is not None:
        _, _, codes = oracle.linear_i8(x, sx, w, sw, bias, so=so)
        _check_codes(got, codes, name)
    else:
        _, ref, _ = oracle.linear_i8(x, sx, w, sw, bias, residual=res)
        _check_bf16(got, ref, x, sx, w, sw, bias, res, name)


def test_linear_i8_ties_round_to_even_and_saturate():
    # x_scale = w_scale = 1, out_scale = 2, no bias: every code is acc / 2
    # exactly, so odd sums are ties (round half to even); out_scale 1/64 on
    # some columns saturates them at +-127 (never -128)
    T, K, N = 64, 64, 64
    _say("linear_i8 ties and saturation")
    x = synth.int8_codes(synth.stream_key(11, 0), T * K, std=3.0).reshape(T, K)
    w = synth.int8_codes(synth.stream_key(11, 1), N * K, std=3.0).reshape(N, K)
    sw = np.ones(N, dtype=np.float32)
    so = np.full(N, 2.0, dtype=np.float32)
    so[:16] = 1.0 / 64
    got = _run(x, 1.0, w, sw, None, None, so)
    acc, _, codes = oracle.linear_i8(x, 1.0, w, sw, None, so=so)
    assert np.count_nonzero(acc[:, 16:] % 2) > 100  # plenty of ties
    _check_codes(got, codes, "ties")
    assert np.array_equal(got[:, 16:], np.clip(np.round(acc[:, 16:] / 2), -127, 127))  # numpy: half even
    assert np.abs(got[:, :16]).max() == 127 and got.min() >= -127


def test_qkv_i8_then_attention_i8():
    # the INT8 chain of the talk: the QKV projection writes INT8 codes with one
    # scale per part, the INT8 attention reads them
    spec = synth.LINEAR_I8_WORKLOADS["qkv-t-s1-i8"]
    a = synth.WORKLOADS["swin-t-s1"]
    B = 4
    T, K, N = B * a["H"] * a["W"], spec["K"], spec["N"]
    nh, M, s = a["heads"], a["window"], a["shifts"][0]
    _say(f"chain qkv-t-s1-i8 -> swin_wattn_fwd_i8, B={B}")
    x, sx, w, sw, bias, _, so = synth.linear_i8_inputs("qkv-t-s1-i8", tokens=T)
    packed = _pack(w)
    qkv = torch.empty(T, N, dtype=torch.int8, device=_dev())
    swa.check(swa.swin_linear_i8_fwd(_i8_dev(x), float(sx), packed, _f32_dev(sw), _f32_dev(bias), None,
                                     _f32_dev(so), qkv, T, K, N), "qkv")
    C = nh * 32
    scales = np.array([so[0], so[C], so[2 * C]], dtype=np.float32)
    assert np.array_equal(so, np.repeat(scales, C))
    table = synth.attention_table(a["seed"], nh, M)
    out = torch.full((B, a["H"], a["W"], C), float("nan"), dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_wattn_fwd_i8(qkv, *(float(v) for v in scales), 0.0, _f32_dev(table), out, B, a["H"],
                                    a["W"], nh, 32, M, s), "attention")
    torch.cuda.synchronize()
    _, _, codes = oracle.linear_i8(x, sx, w, sw, bias, so=so)
    _check_codes(qkv.cpu().numpy(), codes, "qkv codes")
    ref = oracle.swin_wattn_fwd_i8(codes.reshape(B, a["H"], a["W"], 3, nh, 32), scales, table, M, s)
    got = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    print(f"    attention: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
