"""GPU parity of the linear layer (QKV GEMM + bias, output projection + bias
+ residual) against the fp64 oracle, through the C ABI.

Bar, per element: |gpu - oracle| <= 2^-7 |oracle| + 2^-20 (sum_c |x_c w_c| +
|bias| + |residual|).  The output is rounded to nearest-even bf16, whose 8
significant bits give a relative error of at most 2^-8, after an fp32
accumulation of K <= 384 products of exact bf16 inputs (error <= K 2^-24
sum |x w| <= 2^-15.4 sum |x w|, small beside the second term); the bound
takes twice the first.  Inputs are the seeded
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
    lim = 2.0 ** -7 * np.abs(ref) + extra
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


# ------------------------------------------------------- layer norm + linear

def _run_ln(x_bits, gamma, beta, w_bits, bias, eps=1e-5, sel=None):
    T, K = x_bits.shape
    N = w_bits.shape[0]
    w = _bf16_dev(w_bits)
    packed = torch.empty_like(w)
    consts = torch.empty(2, N, dtype=torch.float32, device=_dev())
    g, be = torch.from_numpy(gamma).to(_dev()), torch.from_numpy(beta).to(_dev())
    b = torch.from_numpy(bias).to(_dev()) if bias is not None else None
    swa.check(swa.swin_ln_linear_pack_weight(w, g, be, b, packed, consts, N, K), "ln pack")
    x = _bf16_dev(x_bits)
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_ln_linear_fwd(x, packed, consts, eps, y, T, K, N), "ln_linear")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    if sel is not None:
        y = y[torch.from_numpy(sel).to(_dev())]
    return y.float().cpu().numpy().astype(np.float64)


def _ln_ref_and_bound(x_bits, gamma, beta, w_bits, bias, eps=1e-5):
    """Oracle chain layernorm -> linear in fp64, and the per-element bound:
    the GPU folds gamma into the weight (gamma_c w_jc rounded to bf16,
    relative 2^-8 per element) and beta into the bias (fp32), so beside the
    linear layer's bound it may differ by up to 2^-8 sum_c |z_c gamma_c
    w_c| <= 2^-8 sum_c (|xn_c| + |beta_c|) |w_c| (z the unit-normalised
    row); the bound takes twice that."""
    xn = oracle.layernorm(x_bits, gamma, beta, eps)
    ref = oracle.linear(xn, w_bits, bias)
    w = synth.bf16_to_f32(w_bits).astype(np.float64)
    mag = (np.abs(xn) + np.abs(beta.astype(np.float64))) @ np.abs(w).T
    extra = mag * 2.0 ** -7 + (np.abs(bias.astype(np.float64)) if bias is not None else 0) * 2.0 ** -20
    return ref, extra


@pytest.mark.parametrize("T,K,N,bias", [(1, 32, 32, True), (100, 96, 288, True), (327, 192, 576, True),
                                        (1000, 384, 1152, True), (50, 160, 224, False), (64, 256, 64, True)])
def test_ln_linear_matches_oracle(T, K, N, bias):
    _say(f"ln_linear T={T} K={K} N={N} bias={bias}")
    x, g, be, w, b = synth.make_ln_linear_inputs(T, K, N, seed=T + 3 * K + N)
    b = b if bias else None
    got = _run_ln(x, g, be, w, b)
    ref, extra = _ln_ref_and_bound(x, g, be, w, b)
    _check(got, ref, extra, "ln_linear")


def test_ln_linear_constant_rows_give_beta_projection():
    """A constant token row normalises to beta exactly (zero variance), so the
    output is beta W^T + bias, the folded bias itself."""
    _say("ln_linear constant rows")
    T, K, N = 40, 192, 576
    _, g, be, w, b = synth.make_ln_linear_inputs(T, K, N, seed=5)
    x = synth.bf16_bits(np.repeat(np.linspace(-3, 3, T, dtype=np.float32)[:, None], K, axis=1))
    got = _run_ln(x, g, be, w, b)
    ref, extra = _ln_ref_and_bound(x, g, be, w, b)
    _check(got, ref, extra, "constant rows")


@pytest.mark.parametrize("name", ["lnqkv-t-s1", "lnqkv-t-s3"])
def test_ln_linear_workloads_full(name):
    w_ = synth.LN_LINEAR_WORKLOADS[name]
    _say(f"ln_linear workload {name} full T={w_['tokens']}")
    x, g, be, w, b = synth.ln_linear_inputs(name)
    got = _run_ln(x, g, be, w, b)
    ref, extra = _ln_ref_and_bound(x, g, be, w, b)
    _check(got, ref, extra, name)


def test_ln_linear_full_size_sampled():
    name = "lnqkv-l-s1"
    w_ = synth.LN_LINEAR_WORKLOADS[name]
    _say(f"ln_linear workload {name} full size T={w_['tokens']}, sampled tokens")
    x, g, be, w, b = synth.ln_linear_inputs(name)
    sel = np.sort(np.random.default_rng(6).choice(x.shape[0], 3000, replace=False))
    sel[-1] = x.shape[0] - 1
    got = _run_ln(x, g, be, w, b, sel=sel)
    ref, extra = _ln_ref_and_bound(x[sel], g, be, w, b)
    _check(got, ref, extra, name)


def test_layernorm_qkv_feeds_the_attention():
    """x -> layer norm + QKV GEMM + bias -> fused window attention on the GPU,
    against the fp64 oracle chain, to the attention's bar."""
    B, H, W_, nh, d, M, s = 2, 14, 14, 3, 32, 7, 3
    C = nh * d
    T = B * H * W_
    _say(f"chain LN + QKV -> attention B={B} {H}x{W_} heads={nh} window={M} shift={s}")
    x, g, be, w, b = synth.make_ln_linear_inputs(T, C, 3 * C, seed=98)
    _, table = synth.make_inputs(1, M, M, nh, d, M, seed=98)
    wd = _bf16_dev(w)
    packed = torch.empty_like(wd)
    consts = torch.empty(2, 3 * C, dtype=torch.float32, device=_dev())
    swa.check(swa.swin_ln_linear_pack_weight(wd, torch.from_numpy(g).to(_dev()),
                                             torch.from_numpy(be).to(_dev()),
                                             torch.from_numpy(b).to(_dev()), packed, consts, 3 * C, C),
              "ln pack")
    qkv = torch.empty(T, 3 * C, dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_ln_linear_fwd(_bf16_dev(x), packed, consts, 1e-5, qkv, T, C, 3 * C), "ln_linear")
    out = torch.empty(B, H, W_, C, dtype=torch.bfloat16, device=_dev())
    swa.check(swa.swin_wattn_fwd(qkv, torch.from_numpy(table).to(_dev()), out, B, H, W_, nh, d, M, s),
              "fwd")
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    qkv_ref = oracle.linear(oracle.layernorm(x, g, be), w, b).reshape(B, H, W_, 3, nh, d)
    ref = oracle.swin_wattn_fwd(qkv_ref, table, M, s)
    err = np.abs(got - ref)
    print(f"    chain: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_ln_linear_huge_mean_rows():
    """Rows of mean 1000 and spread 4 (bf16 steps of 4 there): the variance
    is the mean of squared deviations from the mean, as defined; a form
    S2 - S1^2 / K in fp32 would lose about 2 % of it to cancellation (S2 is
    about 1.9e8, K var about 3e3), beyond the bound."""
    _say("ln_linear rows with mean 1000 and spread 4")
    T, K, N = 96, 192, 576
    _, g, be, w, b = synth.make_ln_linear_inputs(T, K, N, seed=22)
    rng = np.random.default_rng(22)
    x = synth.bf16_bits((4.0 * rng.standard_normal((T, K)) + 1000.0).astype(np.float32))
    got = _run_ln(x, g, be, w, b)
    ref, extra = _ln_ref_and_bound(x, g, be, w, b)
    _check(got, ref, extra, "mean 1000")


def test_ln_linear_large_mean_rows():
    """Rows whose mean is large beside their spread: the folded form
    subtracts mean * sum_c W' from the product of the raw row, with the same
    rounded weights on both sides, so the bound needs no extra margin."""
    _say("ln_linear rows with mean 40 and spread 1")
    T, K, N = 96, 192, 576
    _, g, be, w, b = synth.make_ln_linear_inputs(T, K, N, seed=21)
    rng = np.random.default_rng(21)
    x = synth.bf16_bits((rng.standard_normal((T, K)) + 40.0).astype(np.float32))
    got = _run_ln(x, g, be, w, b)
    ref, extra = _ln_ref_and_bound(x, g, be, w, b)
    _check(got, ref, extra, "large mean")
