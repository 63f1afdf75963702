"""GPU parity of the fused attention backward against the fp64 oracle,
through the C ABI.

Bar, per gradient (dq, dk, dv): max-abs error <= 2^-6 of the largest
reference entry and mean-abs error <= 2^-8 of the mean reference magnitude.
The GPU rounds P and dS to bf16 (unit roundoff 2^-8) before the key and
value contractions, and the gradients to bf16 on output; the rest is fp32.
The bias-table gradient (fp32 sums of fp32 dS over every window) is within
1e-3 of its largest entry.  Inputs are seeded
synth.py workloads, and dout is drawn like qkv.  Every case prints its name
before touching the GPU.
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


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(_dev())


def _dout(B, H, W, C, seed):
    return synth.bf16_bits(synth.normal(synth.stream_key(seed, 7), B * H * W * C, 1.0)).reshape(B, H, W, C)


def _run(qkv, table, dout, M, s):
    B, H, W, _, nh, d = qkv.shape
    q, g = _bf16_dev(qkv), _bf16_dev(dout)
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.float32)).to(_dev())
    dq = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=_dev())
    dt = torch.full(t.shape, float("nan"), dtype=torch.float32, device=_dev())
    swa.check(swa.swin_wattn_bwd(q, t, g, dq, dt, B, H, W, nh, d, M, s), "bwd")
    torch.cuda.synchronize()
    return dq.float().cpu().numpy().astype(np.float64), dt.cpu().numpy().astype(np.float64)


def _check(qkv, table, dout, M, s, what):
    dq, dt = _run(qkv, table, dout, M, s)
    rq, rt = oracle.swin_wattn_bwd(qkv, table, dout, M, s)
    assert np.isfinite(dq).all() and np.isfinite(dt).all(), what
    et = np.abs(dt - rt)
    lim_t = 1e-3 * np.abs(rt).max() + 1e-6
    print(f"    {what}: dtable max_err={et.max():.3e} bound {lim_t:.3e}", flush=True)
    bad = []
    for i, name in enumerate("qkv"):
        e = np.abs(dq[:, :, :, i] - rq[:, :, :, i])
        ref = np.abs(rq[:, :, :, i])
        lim_max, lim_mean = 2.0**-6 * ref.max() + 1e-6, 2.0**-8 * ref.mean() + 1e-7
        print(f"      d{name}: max_abs={e.max():.3e} (bound {lim_max:.3e}) "
              f"mean_abs={e.mean():.3e} (bound {lim_mean:.3e}) |ref| max {ref.max():.3f}", flush=True)
        if e.max() > lim_max or e.mean() > lim_mean:
            bad.append(name)
    assert not bad, f"{what}: d{bad}"
    assert et.max() <= lim_t, what


@pytest.mark.parametrize("B,H,W,nh,M,s", [
    (1, 14, 14, 1, 7, 0),     # one head, no shift
    (2, 14, 14, 3, 7, 3),     # shifted: masked windows on the last row and column
    (1, 16, 16, 2, 8, 4),     # window 8: full tiles
    (2, 10, 15, 2, 5, 3),     # window 5: padded tiles, H != W
    (1, 12, 12, 4, 6, 2),
    (2, 8, 8, 2, 4, 2),       # window 4: one tile
    (1, 6, 9, 2, 3, 1),       # window 3: one padded tile
    (1, 4, 4, 1, 2, 1),
    (1, 3, 5, 2, 1, 0),       # window 1: the output is v, so dv = dout, dq = dk = 0
    (1, 7, 14, 48, 7, 3),     # 48 heads, two windows: one window per run
    (3, 14, 14, 5, 7, 3),     # 12 windows, 5 heads: uneven runs
    (1, 24, 24, 2, 12, 6),    # window 12: nine full tiles, one wave per tile
    (2, 24, 36, 3, 12, 5),    # window 12, H != W, odd shift
    (1, 20, 20, 2, 10, 0),    # window 10: padded tiles, no shift
    (1, 18, 27, 1, 9, 4),     # window 9: one padded token row and column per tile row
    (1, 22, 11, 2, 11, 7),    # window 11
    (150, 14, 14, 2, 7, 3),   # window 7, one head per workgroup (head pairs would leave CUs
                              # idle), 600 windows in 75 runs, head pairs placed per XCD
])
def test_backward_matches_oracle(B, H, W, nh, M, s):
    _say(f"bwd B={B} H={H} W={W} nh={nh} M={M} s={s}")
    qkv, table = synth.make_inputs(B, H, W, nh, 32, M, seed=500 + M + s, table_std=0.3)
    dout = _dout(B, H, W, nh * 32, seed=600 + M)
    _check(qkv, table, dout, M, s, f"M={M} s={s}")


@pytest.mark.parametrize("name", ["swin-t-s1", "swin-t-s3"])
def test_backward_workloads(name):
    w = synth.WORKLOADS[name]
    B = min(w["B"], 8)
    qkv, table = synth.workload_inputs(name, batch=B)
    dout = _dout(B, w["H"], w["W"], w["heads"] * w["head_dim"], seed=w["seed"])
    for s in w["shifts"]:
        _say(f"bwd {name} B={B} shift={s}")
        _check(qkv, table, dout, w["window"], s, f"{name} s={s}")


def test_backward_swin_l_sampled_windows():
    """Swin-L stage 1 at B=4 through the GPU; the oracle checks the whole
    output (a few seconds on the host)."""
    w = synth.WORKLOADS["swin-l-s1"]
    qkv, table = synth.workload_inputs("swin-l-s1", batch=4)
    dout = _dout(4, w["H"], w["W"], w["heads"] * 32, seed=w["seed"])
    _say("bwd swin-l-s1 B=4 shift=3")
    _check(qkv, table, dout, 7, 3, "swin-l-s1 B=4")


def test_backward_swin_l_384():
    """Swin-L at 384 px (window 12, shift 6) at B=2: nine tiles per window;
    the oracle checks the whole output."""
    w = synth.WORKLOADS["swin-l-384"]
    qkv, table = synth.workload_inputs("swin-l-384", batch=2)
    dout = _dout(2, w["H"], w["W"], w["heads"] * 32, seed=w["seed"])
    _say("bwd swin-l-384 B=2 shift=6")
    _check(qkv, table, dout, 12, 6, "swin-l-384 B=2")


def test_backward_zero_batch_zeroes_dtable():
    _say("bwd B=0")
    q = torch.empty(0, 14, 14, 3, 2, 32, dtype=torch.bfloat16, device=_dev())
    g = torch.empty(0, 14, 14, 64, dtype=torch.bfloat16, device=_dev())
    t = torch.zeros(169, 2, device=_dev())
    dq = torch.empty(1, 14, 14, 3, 2, 32, dtype=torch.bfloat16, device=_dev())
    dt = torch.full((169, 2), 5.0, device=_dev())
    assert swa.swin_wattn_bwd(q.data_ptr() or 1 << 20, t, g.data_ptr() or 2 << 20, dq, dt, 0, 14, 14,
                              2, 32, 7, 3) == swa.SWIN_OK
    torch.cuda.synchronize()
    assert bool((dt == 0).all())


@pytest.mark.parametrize("name", ["swin-l-s1", "swin-l-384"])
def test_backward_full_size(name):
    """Swin-L stage 1 (B=64, the benchmark's batch and launch configuration)
    and Swin-L at 384 px (B=16, window 12) at full size: the oracle computes
    the whole backward, and dq, dk, dv of every image and the table gradient
    are compared in full."""
    w = synth.WORKLOADS[name]
    B, H, W, nh, M = w["B"], w["H"], w["W"], w["heads"], w["window"]
    s = w["shifts"][-1]
    qkv, table = synth.workload_inputs(name)
    dout = _dout(B, H, W, nh * 32, seed=w["seed"])
    _say(f"bwd {name} full B={B} shift={s}")
    dq, dt = _run(qkv, table, dout, M, s)
    rq, rt = oracle.swin_wattn_bwd(qkv, table, dout, M, s)
    assert np.isfinite(dq).all(), "some gradient was never written (NaN pre-fill) or is not finite"
    assert np.isfinite(dt).all()
    lim_t = 1e-3 * np.abs(rt).max() + 1e-6
    et = np.abs(dt - rt).max()
    print(f"    dtable max_err={et:.3e} bound {lim_t:.3e}", flush=True)
    assert et <= lim_t
    for i, comp in enumerate("qkv"):
        # the bound of each image, on every image
        e = np.abs(dq[:, :, :, i] - rq[:, :, :, i]).reshape(B, -1)
        ref = np.abs(rq[:, :, :, i]).reshape(B, -1)
        emax, emean = e.max(axis=1), e.mean(axis=1)
        lmax, lmean = 2.0**-6 * ref.max(axis=1) + 1e-6, 2.0**-8 * ref.mean(axis=1) + 1e-7
        worst = int(np.argmax(np.maximum(emax / lmax, emean / lmean)))
        print(f"    d{comp}: worst image {worst}: max_abs={emax[worst]:.3e} (bound {lmax[worst]:.3e}) "
              f"mean_abs={emean[worst]:.3e} (bound {lmean[worst]:.3e})", flush=True)
        assert (emax <= lmax).all() and (emean <= lmean).all(), f"d{comp}"


def test_backward_batch_split_over_2gib():
    """600 images of the Swin-L stage-1 shape are 2.17 GB of qkv: the host
    splits the batch into launches of 594 and 6 images (32-bit in-kernel
    offsets).  Eight distinct images (and their output gradients) are tiled
    along the batch on the device, so the gradients of any image are those
    of its source image, and the table gradient is 75 times that of the
    eight (it sums over every image of both launches)."""
    w = synth.WORKLOADS["swin-l-s1"]
    H, W, nh, M, s = w["H"], w["W"], w["heads"], w["window"], w["shifts"][0]
    qkv8, table = synth.workload_inputs("swin-l-s1", batch=8)
    dout8 = _dout(8, H, W, nh * 32, seed=w["seed"])
    B = 600
    _say(f"bwd batch split B={B}")
    q = _bf16_dev(qkv8).repeat(B // 8, 1, 1, 1, 1, 1)
    g = _bf16_dev(dout8).repeat(B // 8, 1, 1, 1)
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.float32)).to(_dev())
    dq = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=_dev())
    dt = torch.full(t.shape, float("nan"), dtype=torch.float32, device=_dev())
    swa.check(swa.swin_wattn_bwd(q, t, g, dq, dt, B, H, W, nh, 32, M, s), "bwd")
    torch.cuda.synchronize()
    rq, rt = oracle.swin_wattn_bwd(qkv8, table, dout8, M, s)
    got_t = dt.cpu().numpy().astype(np.float64)
    ref_t = 75.0 * rt
    et = np.abs(got_t - ref_t).max()
    print(f"    dtable max_err={et:.3e} (|ref| max {np.abs(ref_t).max():.3e})", flush=True)
    assert np.isfinite(got_t).all() and et <= 1e-3 * np.abs(ref_t).max() + 1e-6
    for b in (0, 593, 594, 595, 599):
        got = dq[b].float().cpu().numpy().astype(np.float64)
        for i, comp in enumerate("qkv"):
            e = np.abs(got[:, :, i] - rq[b % 8, :, :, i])
            ref = np.abs(rq[b % 8, :, :, i])
            print(f"    image {b} d{comp}: max_abs={e.max():.3e} mean_abs={e.mean():.3e}", flush=True)
            assert np.isfinite(got).all()
            assert e.max() <= 2.0**-6 * ref.max() + 1e-6 and e.mean() <= 2.0**-8 * ref.mean() + 1e-7
    del q, g, dq
    torch.cuda.empty_cache()
