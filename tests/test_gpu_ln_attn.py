"""GPU parity of the fused layer norm + QKV projection + window attention
(swin_ln_qkv_wattn_fwd) against the fp64 oracle chain layernorm -> linear ->
swin_wattn_fwd, through the C ABI.

Bar: the attention's bf16 tolerances, max-abs <= 2e-2 and mean-abs <= 2e-3,
on every output element.  The GPU rounds gamma o W to bf16 (as
swin_ln_linear_fwd) and q, k, v to bf16 before the attention (as the
two-kernel chain does when it stores qkv); the oracle chain stays in fp64.
Inputs are the seeded layer norm + QKV recipe of synth.py (x = 2 z + 0.5,
gamma = 1 + 0.1 z, beta = 0.1 z, W and bias ~ N(0, 0.02)) with the
attention's bias table.  Every case prints its name before touching the
GPU."""
import numpy as np
import pytest
import torch

import oracle
import shifted_window_attention_swin_amd as swa
import synth

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _dev():
    return torch.device("cuda:0")


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(_dev())


def _run(x, gamma, beta, w, bias, table, M, s, eps=1e-5):
    B, H, W, C = x.shape
    nh = C // 32
    wd = _bf16_dev(w)
    packed = torch.empty_like(wd)
    consts = torch.empty(2, 3 * C, dtype=torch.float32, device=_dev())
    swa.check(swa.swin_ln_linear_pack_weight(wd, torch.from_numpy(gamma).to(_dev()),
                                             torch.from_numpy(beta).to(_dev()),
                                             torch.from_numpy(bias).to(_dev()), packed, consts,
                                             3 * C, C), "pack")
    xd = _bf16_dev(x)
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.float32)).to(_dev())
    out = torch.full((B, H, W, C), float("nan"), dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_ln_qkv_wattn_fwd(xd, packed, consts, eps, t, out, B, H, W, nh, 32, M, s),
              "ln_qkv_wattn")
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item(), "some output position was never written"
    return out.float().cpu().numpy().astype(np.float64)


def _reference(x, gamma, beta, w, bias, table, M, s, eps=1e-5):
    B, H, W, C = x.shape
    xn = oracle.layernorm(x, gamma, beta, eps)
    qkv = oracle.linear(xn, w, bias).reshape(B, H, W, 3, C // 32, 32)
    return oracle.swin_wattn_fwd(qkv, table, M, s)


def _check(got, ref, what):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    print(f"    {what}: max_abs={mx:.3e} mean_abs={mean:.3e} |ref| max {np.abs(ref).max():.3f}",
          flush=True)
    assert np.isfinite(got).all(), what
    assert mx <= MAX_ABS and mean <= MEAN_ABS, what


@pytest.mark.parametrize("B,H,W,nh,M,s", [
    (1, 14, 14, 2, 7, 3),    # shifted: masked windows on the last row and column
    (2, 14, 28, 3, 7, 0),    # H != W, no shift, C = 96 (Swin-T)
    (2, 28, 28, 6, 7, 3),    # C = 192 (Swin-L)
    (1, 16, 16, 4, 8, 4),    # window 8: full tiles, C = 128 (Swin-B)
    (2, 10, 15, 1, 5, 2),    # window 5, one head (C = 32), H != W
    (1, 12, 12, 5, 6, 3),    # window 6, five heads
    (3, 7, 7, 6, 7, 3),      # one window per image covers the image
    (2, 21, 14, 3, 7, 6),    # largest shift
])
def test_ln_attn_matches_oracle_chain(B, H, W, nh, M, s):
    _say(f"ln_qkv_wattn B={B} H={H} W={W} nh={nh} M={M} s={s}")
    x, g, be, w, b, t = synth.make_ln_attn_inputs(B, H, W, nh, M, seed=40 + M + nh + s)
    _check(_run(x, g, be, w, b, t, M, s), _reference(x, g, be, w, b, t, M, s), "chain")


@pytest.mark.parametrize("nh", [3, 6])
def test_ln_attn_huge_mean_rows(nh):
    """Token rows of mean 1000 and spread 4 (bf16 steps of 4 there): the
    statistics lanes must take the variance as the mean of squared
    deviations (the sums S2 and S1 mean nearly cancel).  Three heads run
    4-wave workgroups (one lane per token), six heads 8-wave workgroups
    (two lanes per token, the halves added across the wave)."""
    _say(f"ln_qkv_wattn rows with mean 1000 and spread 4, nh={nh}")
    B, H, W, M, s = 1, 14, 14, 7, 3
    _, g, be, w, b, t = synth.make_ln_attn_inputs(B, H, W, nh, M, seed=70 + nh)
    rng = np.random.default_rng(70 + nh)
    x = synth.bf16_bits((4.0 * rng.standard_normal((B, H, W, 32 * nh)) + 1000.0).astype(np.float32))
    _check(_run(x, g, be, w, b, t, M, s), _reference(x, g, be, w, b, t, M, s), "mean 1000")


@pytest.mark.parametrize("name", ["lnattn-t-s1", "lnattn-l-s1"])
def test_ln_attn_workloads_full_size(name):
    """The launches the benchmark times, every output element against the
    oracle chain."""
    spec = synth.LN_ATTN_WORKLOADS[name]
    a = synth.WORKLOADS[spec["attn"]]
    M, s = a["window"], a["shifts"][0]
    x, g, be, w, b, t = synth.ln_attn_inputs(name)
    _say(f"ln_qkv_wattn {name} full size B={x.shape[0]} shift={s}")
    _check(_run(x, g, be, w, b, t, M, s), _reference(x, g, be, w, b, t, M, s), name)


def test_ln_attn_equals_two_kernel_chain_closely():
    """The fused path and the two-kernel chain (swin_ln_linear_fwd, then
    swin_wattn_fwd) do the same arithmetic except where qkv is rounded in
    the chain's stored qkv and the fused path's LDS tiles (both bf16, both
    from the same fp32 values): the outputs agree to a few bf16 steps."""
    B, H, W, nh, M, s = 2, 28, 28, 6, 7, 3
    _say(f"ln_qkv_wattn against the two-kernel chain B={B} H={H} W={W} nh={nh}")
    x, g, be, w, b, t = synth.make_ln_attn_inputs(B, H, W, nh, M, seed=91)
    C = 32 * nh
    fused = _run(x, g, be, w, b, t, M, s)
    wd = _bf16_dev(w)
    packed = torch.empty_like(wd)
    consts = torch.empty(2, 3 * C, dtype=torch.float32, device=_dev())
    swa.check(swa.swin_ln_linear_pack_weight(wd, torch.from_numpy(g).to(_dev()),
                                             torch.from_numpy(be).to(_dev()),
                                             torch.from_numpy(b).to(_dev()), packed, consts,
                                             3 * C, C), "pack")
    T = B * H * W
    qkv = torch.empty(T, 3 * C, dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_ln_linear_fwd(_bf16_dev(x), packed, consts, 1e-5, qkv, T, C, 3 * C), "ln")
    out = torch.empty(B, H, W, C, dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_wattn_fwd(qkv, torch.from_numpy(t).to(_dev()), out, B, H, W, nh, 32, M, s),
              "fwd")
    torch.cuda.synchronize()
    chain = out.float().cpu().numpy().astype(np.float64)
    d = np.abs(fused - chain)
    print(f"    fused vs chain: max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    assert d.max() <= 1e-2 and d.mean() <= 5e-4


def test_ln_attn_empty_batch_writes_nothing():
    _say("ln_qkv_wattn B=0")
    C = 64
    x = torch.empty(0, 14, 14, C, dtype=torch.bfloat16, device=_dev())
    packed = torch.zeros(3 * C, C, dtype=torch.bfloat16, device=_dev())
    consts = torch.zeros(2, 3 * C, device=_dev())
    t = torch.zeros(169, 2, device=_dev())
    out = torch.full((1, 14, 14, C), 7.0, dtype=torch.bfloat16, device=_dev())
    assert swa.swin_ln_qkv_wattn_fwd(x.data_ptr() or 1 << 20, packed, consts, 1e-5, t, out, 0, 14,
                                     14, 2, 32, 7, 3) == swa.SWIN_OK
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
