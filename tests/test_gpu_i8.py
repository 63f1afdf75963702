"""GPU parity of the INT8 forward (swin_wattn_fwd_i8) against the fp64 oracle,
through the C ABI.

The oracle dequantizes the codes (code times the scale of its part) and runs
the fp64 forward.  Bar: the bf16 forward's (max-abs <= 2e-2, mean-abs <=
2e-3, on outputs of about unit spread: the scales bring the dequantized
values to about N(0, 1)).  At unit scales the INT8 forward is the bf16
forward of the codes taken as bf16 values (exact), so there the two must
agree bit for bit.  Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import shifted_window_attention_swin_amd as swa
import synth

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 2e-3


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _dev():
    return torch.device("cuda:0")


def _run_i8(codes, scales, table, M, s, codes_dev=None, out_scale=0.0):
    B, H, W, _, nh, d = codes.shape
    q = codes_dev if codes_dev is not None else torch.from_numpy(np.ascontiguousarray(codes)).to(_dev())
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.float32)).to(_dev())
    if out_scale > 0:  # -128 is no code: any left is a position never written
        out = torch.full((B, H, W, nh * d), -128, dtype=torch.int8, device=_dev())
    else:
        out = torch.full((B, H, W, nh * d), float("nan"), dtype=torch.bfloat16, device=_dev())
    sq, sk, sv = (float(x) for x in scales)
    swa.check(swa.swin_wattn_fwd_i8(q, sq, sk, sv, float(out_scale), t, out, B, H, W, nh, d, M, s),
              "fwd_i8")
    torch.cuda.synchronize()
    return out


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check(got, ref, what):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    print(f"    {what}: max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert np.isfinite(got).all(), what
    assert mx <= BF16_MAX and mean <= BF16_MEAN, what


@pytest.mark.parametrize("B,H,W,nh,M,s", [
    (2, 14, 14, 6, 7, 3),    # two-head units
    (1, 14, 28, 3, 7, 3),    # three-head units, H != W
    (2, 14, 14, 7, 7, 3),    # one-head units
    (1, 24, 24, 3, 12, 6),   # nine-tile windows
    (2, 8, 8, 4, 4, 2),      # one full tile
    (1, 18, 18, 2, 9, 4),    # ragged tail of 1
])
def test_i8_unit_scales_equal_bf16_of_codes(B, H, W, nh, M, s):
    # the codes are exact in bf16: with scales 1 the INT8 forward must be the
    # bf16 forward of the same values, bit for bit (the loads and the
    # widening are the only difference between the two)
    _say(f"i8 vs bf16 at unit scales B={B} H={H} W={W} nh={nh} M={M} s={s}")
    codes, _, table = synth.make_i8_inputs(B, H, W, nh, 32, M, seed=500 + M + nh)
    a = _run_i8(codes, (1.0, 1.0, 1.0), table, M, s)
    q = torch.from_numpy(codes.astype(np.float32)).to(torch.bfloat16).to(_dev())
    t = torch.from_numpy(table).to(_dev())
    b = torch.full_like(a, float("nan"))
    swa.check(swa.swin_wattn_fwd(q, t, b, B, H, W, nh, 32, M, s), "fwd")
    torch.cuda.synchronize()
    assert not torch.isnan(a).any().item()
    assert torch.equal(a, b)


@pytest.mark.parametrize("B,H,W,nh,M,s", [
    (2, 14, 14, 6, 7, 3),
    (1, 14, 28, 3, 7, 3),    # H != W, three-head units (96-byte slices)
    (2, 28, 14, 2, 7, 0),    # no shift
    (1, 7, 7, 2, 7, 3),      # one window with every region
    (2, 14, 14, 7, 7, 3),    # one-head units
    (4, 14, 14, 4, 7, 3),    # small launch in XCD ranges
    (1, 14, 14, 12, 7, 3),   # many heads per window
    (2, 24, 24, 6, 12, 6),   # window 12, one head's bias per workgroup
    (3, 24, 24, 5, 12, 6),   # window 12, grid cut to keep one head
    (1, 20, 30, 7, 10, 3),
    (1, 22, 11, 3, 11, 5),
    (2, 16, 16, 4, 8, 4),    # four full tiles
    (2, 10, 10, 5, 5, 2),
    (1, 6, 6, 2, 6, 3),
    (2, 6, 4, 2, 2, 1),      # tiny windows
    (1, 3, 3, 1, 1, 0),      # window 1
    (1, 24, 24, 48, 12, 6),  # 48 heads at window 12: tables staged per unit
])
def test_i8_shapes(B, H, W, nh, M, s):
    _say(f"i8 B={B} H={H} W={W} nh={nh} M={M} s={s}")
    codes, scales, table = synth.make_i8_inputs(B, H, W, nh, 32, M, seed=600 + M * 7 + nh)
    got = _f64(_run_i8(codes, scales, table, M, s))
    _check(got, oracle.swin_wattn_fwd_i8(codes, scales, table, M, s), "i8 shape")


@pytest.mark.parametrize("name", ["swin-t-s1-i8", "swin-t-s3-i8", "swin-l-s1-i8", "swin-l-384-i8"])
def test_i8_workloads_full(name):
    # whole workloads at their full batch (the benchmark's launch for
    # swin-l-s1-i8); every output element is compared
    a = synth.WORKLOADS[synth.I8_WORKLOADS[name]["attn"]]
    codes, scales, table = synth.i8_inputs(name)
    for s in a["shifts"]:
        _say(f"i8 {name} full B={a['B']} shift={s}")
        out = _run_i8(codes, scales, table, a["window"], s)
        assert not torch.isnan(out).any().item(), "some output position was never written"
        got = _f64(out)
        del out
        _check(got, oracle.swin_wattn_fwd_i8(codes, scales, table, a["window"], s), f"{name} s={s}")


def test_i8_extreme_codes():
    # every code at -128, -127 or 127: the widening of the ends of the range,
    # sign included
    _say("i8 extreme codes")
    codes, _, table = synth.make_i8_inputs(2, 14, 14, 6, 32, 7, seed=41)
    pick = np.array([-128, -127, 127], dtype=np.int8)
    codes = pick[(codes.astype(np.int64) & 0xFF) % 3]
    scales = np.array([0.004, 0.005, 0.008], dtype=np.float32)
    got = _f64(_run_i8(codes, scales, table, 7, 3))
    _check(got, oracle.swin_wattn_fwd_i8(codes, scales, table, 7, 3), "extreme codes")


@pytest.mark.parametrize("scales", [(0.25, 0.25, 0.03), (1e-4, 1e-4, 0.03), (3e-6, 9e4, 0.03)])
def test_i8_score_scales(scales):
    # a sharp softmax (large query and key scales: weights nearly one-hot), a
    # flat one (tiny scales: the bias and the mask decide), and scales of
    # very different size whose product is moderate
    _say(f"i8 scales {scales}")
    codes, _, table = synth.make_i8_inputs(2, 14, 14, 3, 32, 7, seed=43)
    table = table * np.float32(50.0)  # bias that matters when the scores are flat
    sc = np.array(scales, dtype=np.float32)
    got = _f64(_run_i8(codes, sc, table, 7, 3))
    _check(got, oracle.swin_wattn_fwd_i8(codes, sc, table, 7, 3), f"scales {scales}")


def test_i8_value_scale_is_linear():
    # doubling the value scale doubles every output exactly (a power of two
    # through one fp32 multiply and the bf16 rounding)
    _say("i8 value scale doubling")
    codes, scales, table = synth.make_i8_inputs(2, 14, 14, 3, 32, 7, seed=47)
    a = _run_i8(codes, scales, table, 7, 3)
    b = _run_i8(codes, (scales[0], scales[1], scales[2] * 2), table, 7, 3)
    assert torch.equal(b.float(), 2.0 * a.float())


def test_i8_repeatable_bit_exact():
    _say("i8 repeatability")
    codes, scales, table = synth.make_i8_inputs(4, 28, 28, 6, 32, 7, seed=49)
    a = _run_i8(codes, scales, table, 7, 3)
    b = _run_i8(codes, scales, table, 7, 3)
    assert torch.equal(a, b)


def test_i8_batch_split_over_2gib():
    # 1200 images of the Swin-L stage-1 shape are 2.17 GB of int8 qkv: the
    # host splits the batch at 1188 images.  Eight distinct images are tiled
    # along the batch; windows on both sides of the split are checked against
    # the oracle of their source image.
    a = synth.WORKLOADS["swin-l-s1"]
    H, W, nh, M, s = a["H"], a["W"], a["heads"], a["window"], a["shifts"][0]
    codes8, scales, table = synth.i8_inputs("swin-l-s1-i8", batch=8)
    B = 1200
    _say(f"i8 batch split B={B}")
    q = torch.from_numpy(codes8).to(_dev()).repeat(B // 8, 1, 1, 1, 1, 1)
    # the host array only gives the shape: the codes are the device copy
    shape_only = np.broadcast_to(codes8[:1], (B, H, W, 3, nh, 32))
    out = _run_i8(shape_only, scales, table, M, s, codes_dev=q)
    assert not torch.isnan(out).any().item()
    x = oracle.dequant_qkv_i8(codes8, scales)
    nW = (H // M) * (W // M)
    images = [0, 1187, 1188, 1189, 1199]
    sel = np.array([(b % 8) * nW + wi for b in images for wi in (0, 7, 56, 63, 27)], dtype=np.int64)
    ref, pos = oracle.swin_wattn_windows(x, table, M, s, sel)
    k = 0
    for b in images:
        for _ in range(5):
            idx = torch.from_numpy(pos[k] + (b - b % 8) * H * W).to(_dev())
            _check(_f64(out.view(B * H * W, nh * 32)[idx]), ref[k], f"image {b}")
            k += 1
    del q, out
    torch.cuda.empty_cache()


def _check_out_codes(got, o64, so, what, min_equal=0.97):
    # int8 output: the code rounds the fp32 output, whose error against the
    # fp64 value is the bf16 path's (weights rounded to bf16) without the
    # output rounding.  Every code must be within 1 of the fp64 value's
    # code (round half to even, clamped), nearly all equal to it, and codes
    # far beyond the range saturate
    exact = np.clip(np.rint(o64 / so), -127, 127)
    d = np.abs(got.astype(np.float64) - exact)
    eq = float(np.mean(d == 0))
    print(f"    {what}: max code diff {d.max():.0f}, equal {eq:.4f}, saturated "
          f"{np.mean(np.abs(exact) == 127):.4f}", flush=True)
    assert d.max() <= 1 and eq >= min_equal, what
    far = np.abs(o64 / so) > 128
    assert np.array_equal(got[far], 127 * np.sign(o64[far])), what


@pytest.mark.parametrize("B,H,W,nh,M,s", [(4, 56, 56, 6, 7, 3), (2, 24, 24, 3, 12, 6), (2, 14, 14, 7, 7, 3)])
def test_i8_int8_output(B, H, W, nh, M, s):
    _say(f"i8 int8 output B={B} H={H} W={W} nh={nh} M={M} s={s}")
    codes, scales, table = synth.make_i8_inputs(B, H, W, nh, 32, M, seed=660 + M + nh)
    o64 = oracle.swin_wattn_fwd_i8(codes, scales, table, M, s)
    so = float(np.float32(np.abs(o64).max() / 127.0))
    out = _run_i8(codes, scales, table, M, s, out_scale=so)
    got = out.cpu().numpy()
    assert (got != -128).all(), "some output position was never written"
    _check_out_codes(got, o64, so, "codes")


def test_i8_int8_output_saturates():
    _say("i8 int8 output saturation")
    codes, scales, table = synth.make_i8_inputs(2, 14, 14, 6, 32, 7, seed=671)
    o64 = oracle.swin_wattn_fwd_i8(codes, scales, table, 7, 3)
    so = float(np.float32(np.quantile(np.abs(o64), 0.7) / 127.0))  # about 30% beyond +-127
    got = _run_i8(codes, scales, table, 7, 3, out_scale=so).cpu().numpy()
    _check_out_codes(got, o64, so, "saturating codes", min_equal=0.9)
    assert np.mean(np.abs(got) == 127) > 0.1 and got.min() >= -127


def test_int8_block_chain():
    # QKV projection (INT8 out) -> attention (INT8 in, INT8 out) -> output
    # projection (INT8 in, bf16 out, + bias + residual): each stage against
    # the oracle on the codes the previous GPU stage wrote
    spec = synth.LINEAR_I8_WORKLOADS["qkv-l-s1-i8"]
    a = synth.WORKLOADS["swin-l-s1"]
    B = 2
    H, W, nh, M, s = a["H"], a["W"], a["heads"], a["window"], a["shifts"][0]
    C = nh * 32
    T = B * H * W
    _say(f"INT8 block chain, Swin-L stage 1 shape, B={B}")
    x, sx, w, sw, bias, _, so = synth.linear_i8_inputs("qkv-l-s1-i8", tokens=T)
    dev = _dev()
    f32 = lambda v: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(dev)
    packed = torch.zeros(3 * C * ((C + 63) // 64) * 64, dtype=torch.int8, device=dev)
    swa.check(swa.swin_linear_i8_pack_weight(torch.from_numpy(w).to(dev), packed, 3 * C, C), "pack")
    qkv = torch.full((T, 3 * C), -128, dtype=torch.int8, device=dev)
    swa.check(swa.swin_linear_i8_fwd(torch.from_numpy(x).to(dev), float(sx), packed, f32(sw), f32(bias),
                                     None, f32(so), qkv, T, C, 3 * C), "qkv")
    scales = np.array([so[0], so[C], so[2 * C]], dtype=np.float32)
    table = synth.attention_table(a["seed"], nh, M)
    qkv_codes = qkv.cpu().numpy()
    _, _, ref_qkv = oracle.linear_i8(x, sx, w, sw, bias, so=so)
    assert np.array_equal(qkv_codes, ref_qkv)
    o64 = oracle.swin_wattn_fwd_i8(qkv_codes.reshape(B, H, W, 3, nh, 32), scales, table, M, s)
    so_attn = float(np.float32(np.abs(o64).max() / 127.0))
    att = _run_i8(qkv_codes.reshape(B, H, W, 3, nh, 32), scales, table, M, s, codes_dev=qkv,
                  out_scale=so_attn)
    att_codes = att.cpu().numpy()
    _check_out_codes(att_codes, o64, so_attn, "attention codes")
    # the output projection on the attention's codes
    _, _, w2, sw2, b2, res, _ = synth.make_linear_i8_inputs(T, C, C, 2103, True, False)
    packed2 = torch.zeros(C * ((C + 63) // 64) * 64, dtype=torch.int8, device=dev)
    swa.check(swa.swin_linear_i8_pack_weight(torch.from_numpy(w2).to(dev), packed2, C, C), "pack2")
    y = torch.from_numpy(res.view(np.int16)).view(torch.bfloat16).to(dev).clone()
    swa.check(swa.swin_linear_i8_fwd(att.view(T, C), so_attn, packed2, f32(sw2), f32(b2), y, None, y,
                                     T, C, C), "proj")
    torch.cuda.synchronize()
    _, ref, _ = oracle.linear_i8(att_codes.reshape(T, C), so_attn, w2, sw2, b2, residual=res)
    got = y.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert (err <= 2.0 ** -7 * np.abs(ref) + 1e-3).all(), float(err.max())
