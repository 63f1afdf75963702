"""GPU parity of libswinattn against the fp64 oracle, through the C ABI.

Bar: bf16 max-abs <= 2e-2 and mean-abs <= 2e-3; fp32 max-abs <= 1e-4;
precomputed index / mask / region labels bit-exact.  Inputs are the seeded
workloads of synth.py, read identically by both sides.  Every case prints its
name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import shifted_window_attention_swin_amd as swa
import synth

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _dev():
    return torch.device("cuda:0")


def _to_dev(qkv):
    if qkv.dtype == np.uint16:
        return torch.from_numpy(qkv.view(np.int16)).view(torch.bfloat16).to(_dev())
    return torch.from_numpy(np.ascontiguousarray(qkv, dtype=np.float32)).to(_dev())


def _run(qkv, table, M, s, out=None):
    """One forward on the GPU; returns the device output tensor."""
    B, H, W, _, nh, d = qkv.shape
    q = _to_dev(qkv)
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.float32)).to(_dev())
    if out is None:
        out = torch.full((B, H, W, nh * d), float("nan"), dtype=q.dtype, device=_dev())
    fn = swa.swin_wattn_fwd if q.dtype == torch.bfloat16 else swa.swin_wattn_fwd_f32
    swa.check(fn(q, t, out, B, H, W, nh, d, M, s), "fwd")
    torch.cuda.synchronize()
    return out


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check(got, ref, bf16, what):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    print(f"    {what}: max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert np.isfinite(got).all(), what
    if bf16:
        assert mx <= BF16_MAX and mean <= BF16_MEAN, what
    else:
        assert mx <= F32_MAX, what


# ------------------------------------------------------------- precompute

@pytest.mark.parametrize("H,W,M,s", [(14, 14, 7, 3), (56, 56, 7, 3), (14, 14, 7, 0), (96, 96, 12, 6),
                                     (4, 4, 2, 1), (28, 14, 7, 2), (24, 36, 12, 5), (7, 7, 7, 3)])
def test_precompute_bit_exact(H, W, M, s):
    _say(f"precompute H={H} W={W} M={M} s={s}")
    swa.check(swa.swin_wattn_precompute(H, W, M, s))
    N, nW = M * M, (H // M) * (W // M)
    idx = torch.empty(N, N, dtype=torch.int32, device=_dev())
    mask = torch.empty(nW, N, N, dtype=torch.float32, device=_dev())
    reg = torch.empty(nW, N, dtype=torch.uint8, device=_dev())
    swa.check(swa.swin_wattn_copy_index(H, W, M, s, idx))
    swa.check(swa.swin_wattn_copy_mask(H, W, M, s, mask))
    swa.check(swa.swin_wattn_copy_region(H, W, M, s, reg))
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), oracle.rel_index(M))
    assert np.array_equal(mask.cpu().numpy(), oracle.shift_mask(H, W, M, s).astype(np.float32))
    lab = oracle.window_partition(oracle.region_labels(H, W, M, s)[None, :, :, None].astype(np.float64), M)
    assert np.array_equal(reg.cpu().numpy().astype(np.float64), lab.reshape(nW, N))


def test_precompute_copy_on_another_stream():
    """The fill is queued on one stream and the copies on another, with no
    host synchronisation between them: the copy stream waits for the event
    the precompute recorded, so the copies see the finished tensors."""
    H, W, M, s = 96, 96, 12, 6
    _say(f"precompute on stream A, copies on stream B, H={H} W={W} M={M} s={s}")
    swa.check(swa.swin_wattn_release())
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    N, nW = M * M, (H // M) * (W // M)
    mask = torch.full((nW, N, N), float("nan"), dtype=torch.float32, device=_dev())
    idx = torch.full((N, N), -1, dtype=torch.int32, device=_dev())
    torch.cuda.synchronize()
    swa.check(swa.swin_wattn_precompute(H, W, M, s, a))
    swa.check(swa.swin_wattn_copy_mask(H, W, M, s, mask, b))
    swa.check(swa.swin_wattn_copy_index(H, W, M, s, idx, b))
    b.synchronize()
    assert np.array_equal(mask.cpu().numpy(), oracle.shift_mask(H, W, M, s).astype(np.float32))
    assert np.array_equal(idx.cpu().numpy(), oracle.rel_index(M))
    torch.cuda.synchronize()
    swa.check(swa.swin_wattn_release())


# ---------------------------------------------------------------- fp32

def test_fp32_tiny_workload():
    _say("fp32 tiny-f32 B=1 14x14 nh=2 M=7 s=3")
    qkv, table = synth.workload_inputs("tiny-f32")
    got = _f64(_run(qkv, table, 7, 3))
    _check(got, oracle.swin_wattn_fwd(qkv, table, 7, 3), False, "tiny-f32")


@pytest.mark.parametrize("B,H,W,nh,M,s", [(2, 28, 14, 3, 7, 0), (1, 24, 24, 2, 12, 6), (2, 8, 8, 1, 4, 2),
                                          (1, 10, 15, 2, 5, 4)])
def test_fp32_shapes(B, H, W, nh, M, s):
    _say(f"fp32 B={B} H={H} W={W} nh={nh} M={M} s={s}")
    qkv, table = synth.make_inputs(B, H, W, nh, 32, M, seed=31 + M, dtype="f32")
    got = _f64(_run(qkv, table, M, s))
    _check(got, oracle.swin_wattn_fwd(qkv, table, M, s), False, "fp32 shape")


# ---------------------------------------------------------------- bf16

@pytest.mark.parametrize("name", ["swin-t-s1", "swin-t-s3"])
def test_bf16_workloads_full(name):
    w = synth.WORKLOADS[name]
    qkv, table = synth.workload_inputs(name)
    for s in w["shifts"]:
        _say(f"bf16 {name} full B={w['B']} shift={s}")
        got = _f64(_run(qkv, table, w["window"], s))
        _check(got, oracle.swin_wattn_fwd(qkv, table, w["window"], s), True, f"{name} s={s}")


@pytest.mark.parametrize("name,batch", [("swin-l-s1", 4), ("swin-l-384", 2)])
def test_bf16_workloads_small_batch_full(name, batch):
    w = synth.WORKLOADS[name]
    qkv, table = synth.workload_inputs(name, batch=batch)
    s = w["shifts"][0]
    _say(f"bf16 {name} B={batch} shift={s}")
    got = _f64(_run(qkv, table, w["window"], s))
    _check(got, oracle.swin_wattn_fwd(qkv, table, w["window"], s), True, f"{name} B={batch}")


@pytest.mark.parametrize("name", ["swin-l-s1", "swin-l-384"])
def test_bf16_workloads_full_size(name):
    # the launch the benchmark times: full batch; the oracle computes the
    # whole forward (a second or two on the host) and every output element
    # is compared
    w = synth.WORKLOADS[name]
    B, H, W, nh, M = w["B"], w["H"], w["W"], w["heads"], w["window"]
    s = w["shifts"][0]
    qkv, table = synth.workload_inputs(name)
    _say(f"bf16 {name} full size B={B} shift={s}")
    out = _run(qkv, table, M, s)
    assert not torch.isnan(out).any().item(), "some output position was never written"
    got = _f64(out)
    del out
    _check(got, oracle.swin_wattn_fwd(qkv, table, M, s), True, f"{name} every window")


@pytest.mark.parametrize("B,H,W,nh,M,s", [
    (1, 14, 28, 3, 7, 3),    # H != W
    (2, 28, 14, 6, 7, 3),
    (1, 7, 7, 2, 7, 0),      # one window covers the image, no shift
    (1, 7, 7, 2, 7, 3),      # one window with shift: every region in one window
    (1, 12, 12, 6, 12, 0),   # 6 units on 6 workgroups (grid order), one head's bias each
    (2, 24, 24, 6, 12, 6),   # 48 units, XCD ranges: every workgroup keeps one head
    (3, 24, 24, 5, 12, 6),   # 60 units: the grid is cut from 56 to 40 to keep one head
    (1, 20, 30, 7, 10, 3),   # 42 units, grid 40 < 8 x 7: every head's bias staged
    (2, 12, 24, 1, 12, 5),   # one head
    (3, 8, 8, 1, 4, 2),      # N = 16: one full tile
    (2, 16, 16, 4, 8, 4),    # N = 64: four full tiles
    (2, 10, 10, 5, 5, 2),    # odd head count
    (1, 18, 18, 2, 9, 4),    # N = 81: ragged tail of 1
    (1, 22, 11, 3, 11, 5),   # N = 121
    (1, 6, 6, 2, 6, 3),      # N = 36
    (2, 6, 4, 2, 2, 1),      # tiny windows
    (1, 3, 3, 1, 1, 0),      # window 1: each token attends to itself
    (2, 14, 14, 7, 7, 3),    # 7 heads: one-head units, grid cut to 8 x 7 with XCD ranges
    (4, 14, 14, 4, 7, 3),    # 4 heads: two-head units, a small launch in XCD ranges
    (1, 14, 14, 12, 7, 3),   # many heads per window
    (1, 14, 14, 16, 7, 0),
])
def test_bf16_shapes(B, H, W, nh, M, s):
    _say(f"bf16 B={B} H={H} W={W} nh={nh} M={M} s={s}")
    qkv, table = synth.make_inputs(B, H, W, nh, 32, M, seed=100 + M * 7 + nh, dtype="bf16")
    got = _f64(_run(qkv, table, M, s))
    _check(got, oracle.swin_wattn_fwd(qkv, table, M, s), True, "bf16 shape")


def test_bf16_large_bias_and_mask_dominate():
    # bias of std 3 makes the bias term decide the weights: catches a bias
    # gathered for the wrong (query, key) pair or head on the GPU
    _say("bf16 large bias table std 3")
    qkv, table = synth.make_inputs(2, 14, 14, 3, 32, 7, seed=7, dtype="bf16", table_std=3.0)
    got = _f64(_run(qkv, table, 7, 3))
    _check(got, oracle.swin_wattn_fwd(qkv, table, 7, 3), True, "large bias")


def test_window_one_returns_value():
    _say("bf16 window 1")
    qkv, table = synth.make_inputs(2, 5, 3, 2, 32, 1, seed=3, dtype="bf16")
    got = _run(qkv, table, 1, 0)
    v = torch.from_numpy(qkv.view(np.int16)).view(torch.bfloat16)[:, :, :, 2].reshape(2, 5, 3, 64)
    assert torch.equal(got.cpu(), v)


# ------------------------------------------------------ exact properties

def test_value_doubling_is_exact_on_gpu():
    _say("bf16 linearity in v")
    qkv, table = synth.make_inputs(2, 14, 14, 3, 32, 7, seed=17, dtype="bf16")
    a = _run(qkv, table, 7, 3)
    q2 = qkv.copy()
    q2[:, :, :, 2] = synth.bf16_bits(synth.bf16_to_f32(qkv[:, :, :, 2]) * 2.0)
    b = _run(q2, table, 7, 3)
    assert torch.equal(b.float(), 2.0 * a.float())


def test_repeatable_bit_exact():
    _say("bf16 repeatability")
    qkv, table = synth.make_inputs(4, 28, 28, 6, 32, 7, seed=19, dtype="bf16")
    a = _run(qkv, table, 7, 3)
    b = _run(qkv, table, 7, 3)
    assert torch.equal(a, b)


def test_empty_batch_writes_nothing():
    _say("bf16 B=0")
    q = torch.empty(0, 14, 14, 3, 2, 32, dtype=torch.bfloat16, device=_dev())
    t = torch.zeros(169, 2, device=_dev())
    out = torch.full((1, 14, 14, 64), 7.0, dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_wattn_precompute(14, 14, 7, 3))
    assert swa.swin_wattn_fwd(q.data_ptr() or 1 << 20, t, out, 0, 14, 14, 2, 32, 7, 3) == swa.SWIN_OK
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_needs_no_setup_and_release(dtype):
    """The forward evaluates index and mask itself: it runs, and matches the
    oracle, with nothing prepared; only the copy calls need the precompute."""
    _say(f"forward without precompute / release, {dtype}")
    swa.check(swa.swin_wattn_release())
    qkv, table = synth.make_inputs(2, 22, 22, 3, 32, 2, seed=1234, dtype=dtype)
    got = _f64(_run(qkv, table, 2, 1))
    _check(got, oracle.swin_wattn_fwd(qkv, table, 2, 1), dtype == "bf16", "no precompute")
    idx = torch.empty(16, dtype=torch.int32, device=_dev())
    assert swa.swin_wattn_copy_index(22, 22, 2, 1, idx) == swa.SWIN_ERR_NOT_PREPARED
    swa.check(swa.swin_wattn_precompute(22, 22, 2, 1))
    swa.check(swa.swin_wattn_copy_index(22, 22, 2, 1, idx))
    again = _f64(_run(qkv, table, 2, 1))
    assert np.array_equal(got, again)
    swa.check(swa.swin_wattn_release())
    assert swa.swin_wattn_copy_index(22, 22, 2, 1, idx) == swa.SWIN_ERR_NOT_PREPARED


@pytest.mark.parametrize("B,H,W,nh,M,s", [
    # every head's bias tables beyond the 64 KiB staged per workgroup: each
    # workgroup stages one head group's tables, fixed for its units when the
    # grid allows it, else staged again whenever the unit's group changes
    (16, 12, 12, 32, 12, 0),  # Swin-B at 384 px, stage 4 (window = image): fixed group
    (16, 12, 12, 48, 12, 0),  # Swin-L at 384 px, stage 4: fixed group
    (1, 12, 12, 48, 12, 0),   # 48 units on 48 workgroups: restaged
    (2, 24, 24, 48, 12, 6),   # shifted, 4 windows, restaged
    (1, 14, 14, 64, 7, 3),    # two-head units of 64 heads: restaged
    (1, 24, 24, 20, 12, 6),
])
def test_bf16_many_heads(B, H, W, nh, M, s):
    _say(f"bf16 many heads B={B} H={H} W={W} nh={nh} M={M} s={s}")
    qkv, table = synth.make_inputs(B, H, W, nh, 32, M, seed=300 + nh, dtype="bf16")
    got = _f64(_run(qkv, table, M, s))
    _check(got, oracle.swin_wattn_fwd(qkv, table, M, s), True, "bf16 many heads")


def test_bf16_batch_split_over_2gib():
    # 600 images of the Swin-L stage-1 shape are 2.17 GB of qkv: the host
    # splits the batch at 594 images (32-bit in-kernel offsets).  Eight
    # distinct images are tiled along the batch on the device; windows on both
    # sides of the split are checked against the oracle of their source image.
    w = synth.WORKLOADS["swin-l-s1"]
    H, W, nh, M, s = w["H"], w["W"], w["heads"], w["window"], w["shifts"][0]
    qkv8, table = synth.workload_inputs("swin-l-s1", batch=8)
    B = 600
    _say(f"bf16 batch split B={B}")
    q8 = _to_dev(qkv8)
    q = q8.repeat(B // 8, 1, 1, 1, 1, 1)
    t = torch.from_numpy(table).to(_dev())
    out = torch.full((B, H, W, nh * 32), float("nan"), dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_wattn_precompute(H, W, M, s))
    swa.check(swa.swin_wattn_fwd(q, t, out, B, H, W, nh, 32, M, s))
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item()
    nW = (H // M) * (W // M)
    images = [0, 593, 594, 595, 599]
    sel = np.array([(b % 8) * nW + wi for b in images for wi in (0, 7, 56, 63, 27)], dtype=np.int64)
    ref, pos = oracle.swin_wattn_windows(qkv8, table, M, s, sel)
    k = 0
    for b in images:
        for _ in range(5):
            got = _f64(out.view(B * H * W, nh * 32)[torch.from_numpy(pos[k] + (b - b % 8) * H * W).to(_dev())])
            _check(got, ref[k], True, f"image {b}")
            k += 1
    del q, out
    torch.cuda.empty_cache()
