"""GPU parity of the linear layer (QKV GEMM + bias, output projection + bias
+ residual) against the fp64 oracle, through the C ABI.

Bar, per element: |gpu - oracle| <= 2^-8 |oracle| + 2^-20 (sum_c |x_c w_c| +
|bias| + |residual|).  The output is rounded to nearest-even bf16 (relative
error <= 2^-9) after an fp32 accumulation of K <= 384 products of exact bf16
inputs (error <= K 2^-24 sum |x w| <= 2^-15.4 sum |x w|); the bound takes
twice the first and more than twice the second.  Inputs are the seeded
workloads of synth.py.  Every case prints its name before touching the GPU.
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


def _pack(w_bits):
    N, K = w_bits.shape
    w = _bf16_dev(w_bits)
    packed = torch.empty_like(w)
    swa.check(swa.swin_linear_pack_weight(w, packed, N, K), "pack")
    return packed


def _run(x_bits, w_bits, bias, res_bits, inplace=False, sel=None):
    T, K = x_bits.shape
    N = w_bits.shape[0]
    packed = _pack(w_bits)
    x = _bf16_dev(x_bits)
    b = torch.from_numpy(bias).to(_dev()) if bias is not None else None
    if inplace:
        y = _bf16_dev(res_bits)
        r = y
    else:
        r = _bf16_dev(res_bits) if res_bits is not None else None
        y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_linear_fwd(x, packed, b, r, y, T, K, N), "linear")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    if sel is not None:
        y = y[torch.from_numpy(sel).to(_dev())]
    return y.float().cpu().numpy().astype(np.float64)


def _bound(x_bits, w_bits, bias, res_bits):
    x = synth.bf16_to_f32(x_bits).astype(np.float64)
    w = synth.bf16_to_f32(w_bits).astype(np.float64)
    mag = np.abs(x) @ np.abs(w).T
    if bias is not None:
        mag = mag + np.abs(bias.astype(np.float64))
    if res_bits is not None:
        mag = mag + np.abs(synth.bf16_to_f32(res_bits).astype(np.float64))
    return mag * 2.0 ** -20


def _check(got, ref, extra, what):
    err = np.abs(got - ref)
    lim = 2.0 ** -8 * np.abs(ref) + extra
    worst = float((err / lim).max()) if err.size else 0.0
    print(f"    {what}: max_abs={err.max() if err.size else 0:.3e} worst err/bound={worst:.3f}",
          flush=True)
    assert np.isfinite(got).all(), what
    assert (err <= lim).all(), what


@pytest.mark.parametrize("T,K,N,bias,res", [
    (1, 32, 32, True, False),        # one token, one k-step, one column block
    (16, 64, 96, False, False),      # no bias
    (100, 96, 288, True, False),     # Swin-T QKV shape, ragged last row block
    (64 * 5 + 7, 192, 576, True, False),   # Swin-L QKV shape, ragged
    (1000, 384, 1152, True, False),  # Swin-T stage 3 QKV shape, two weight chunks
    (777, 192, 192, True, True),     # output projection + residual
    (513, 384, 384, True, True),
    (300, 160, 224, True, True),     # K, N not multiples of 64 / 96
])
def test_linear_matches_oracle(T, K, N, bias, res):
    _say(f"linear T={T} K={K} N={N} bias={bias} residual={res}")
    x, w, b, r = synth.make_linear_inputs(T, K, N, seed=T + K + N, residual=res)
    b = b if bias else None
    got = _run(x, w, b, r)
    ref = oracle.linear(x, w, b, r)
    _check(got, ref, _bound(x, w, b, r), "linear")


def test_linear_in_place_residual():
    _say("linear in-place residual (residual == y)")
    x, w, b, r = synth.make_linear_inputs(200, 192, 192, seed=77, residual=True)
    got = _run(x, w, b, r, inplace=True)
    _check(got, oracle.linear(x, w, b, r), _bound(x, w, b, r), "in place")


@pytest.mark.parametrize("name", ["qkv-t-s1", "qkv-t-s3", "proj-t-s3"])
def test_linear_workloads_full(name):
    w_ = synth.LINEAR_WORKLOADS[name]
    _say(f"linear workload {name} full T={w_['tokens']}")
    x, w, b, r = synth.linear_inputs(name)
    got = _run(x, w, b, r)
    _check(got, oracle.linear(x, w, b, r), _bound(x, w, b, r), name)


@pytest.mark.parametrize("name", ["qkv-l-s1", "proj-l-s1"])
def test_linear_workloads_full_size_sampled(name):
    """Full size, in the launch configuration the benchmark times; the oracle
    recomputes 3000 sampled tokens (every column)."""
    w_ = synth.LINEAR_WORKLOADS[name]
    _say(f"linear workload {name} full size T={w_['tokens']}, sampled tokens")
    x, w, b, r = synth.linear_inputs(name)
    sel = np.sort(np.random.default_rng(5).choice(x.shape[0], 3000, replace=False))
    sel[-1] = x.shape[0] - 1
    got = _run(x, w, b, r, sel=sel)
    rs = r[sel] if r is not None else None
    ref = oracle.linear(x[sel], w, b, rs)
    _check(got, ref, _bound(x[sel], w, b, rs), name)


def test_qkv_projection_feeds_the_attention():
    """The chain x -> QKV GEMM + bias -> fused window attention on the GPU
    against the fp64 oracle chain, to the attention's bar (the GPU rounds qkv
    to bf16 between the two)."""
    B, H, W_, nh, d, M, s = 2, 14, 14, 3, 32, 7, 3
    C = nh * d
    T = B * H * W_
    _say(f"chain QKV -> attention B={B} {H}x{W_} heads={nh} window={M} shift={s}")
    x, w, b, _ = synth.make_linear_inputs(T, C, 3 * C, seed=99, residual=False)
    _, table = synth.make_inputs(1, M, M, nh, d, M, seed=99)
    packed = _pack(w)
    xd = _bf16_dev(x)
    qkv = torch.empty(T, 3 * C, dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_linear_fwd(xd, packed, torch.from_numpy(b).to(_dev()), None, qkv, T, C,
                                  3 * C), "linear")
    out = torch.empty(B, H, W_, C, dtype=torch.bfloat16, device=_dev())
    t = torch.from_numpy(table).to(_dev())
    swa.check(swa.swin_wattn_fwd(qkv, t, out, B, H, W_, nh, d, M, s), "fwd")
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    qkv_ref = oracle.linear(x, w, b).reshape(B, H, W_, 3, nh, d)
    ref = oracle.swin_wattn_fwd(qkv_ref, table, M, s)
    err = np.abs(got - ref)
    print(f"    chain: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_linear_empty_writes_nothing():
    _say("linear T=0")
    y = torch.full((4, 64), 7.0, dtype=torch.bfloat16, device=_dev())
    w = torch.zeros(64, 32, dtype=torch.bfloat16, device=_dev())
    x = torch.zeros(4, 32, dtype=torch.bfloat16, device=_dev())
    assert swa.swin_linear_fwd(x, w, None, None, y, 0, 32, 64) == swa.SWIN_OK
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
