"""Benchmark of the fused shifted-window attention forward on one MI355X.

A step is one ``swin_wattn_fwd`` over the whole batch of the workload (default:
Swin-L stage 1, B=64, 56x56 tokens, 6 heads x 32, window 7, shift 3, bf16)
with inputs already resident in HBM.  Input/output buffer sets rotate so that
the working set of the timed region exceeds twice the 256 MB Infinity Cache
(cold cache).  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

With --backward a step is one swin_wattn_bwd over the workload instead (the
bias-gradient zero fill and the backward kernel).  With --workload naming a
linear-layer workload (qkv-l-s1, proj-l-s1, ...) a
step is one swin_linear_fwd over its tokens instead, with a layer norm +
QKV workload (lnqkv-l-s1, ...) one swin_ln_linear_fwd, and with a layer norm
+ attention workload (lnattn-l-s1, lnattn-t-s1) one swin_ln_qkv_wattn_fwd
(the two-kernel chain is timed beside it).  With an INT8 attention workload
(swin-l-s1-i8, ...) a step is one swin_wattn_fwd_i8 over the workload, and
with an INT8 linear workload (qkv-l-s1-i8, ...) one swin_linear_i8_fwd.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "shifted-window attn fwd GB/s & TFLOP/s (Swin-L stage1, bf16, B=64); % HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
MALL_BYTES = 256 * 2 ** 20
CSRC = os.path.join(ROOT, "shifted_window_attention_swin_amd", "csrc")


# the sources that define each kernel family's device code
KERNEL_SOURCES = {
    "wattn_fwd_bf16": ("wattn_internal.h", "wattn_common.h", "wattn_persistent.hip"),
    "wattn_fwd_i8": ("wattn_internal.h", "wattn_common.h", "wattn_persistent.hip"),
    "ln_qkv_wattn": ("wattn_internal.h", "wattn_common.h", "ln_attn_internal.h", "ln_qkv_wattn.hip"),
    "linear_fwd": ("wattn_internal.h", "wattn_common.h", "linear_internal.h", "linear_gemm.hip"),
    "wattn_bwd_bf16": ("wattn_internal.h", "wattn_common.h", "bwd_internal.h", "wattn_backward.hip"),
}


def kernel_source_hash(family: str = "wattn_fwd_bf16") -> str:
    """Hash of the sources of a kernel family: a committed traffic
    measurement is only reported while the sources it was taken on are
    unchanged."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic(B, H, W, heads, head_dim, window, elem=2, out_elem=None):
    """Bytes: qkv read once (`elem` bytes per element) + out written once
    (`out_elem`, default `elem`).  FLOPs: two contractions of N x N x
    head_dim per window and head over the unpadded N."""
    T = B * H * W
    C = heads * head_dim
    N = window * window
    out_elem = elem if out_elem is None else out_elem
    return 3 * C * T * elem + C * T * out_elem, 4 * N * C * T


def bwd_algorithmic(B, H, W, heads, head_dim, window, elem=2):
    """Bytes: qkv and dout read once, dqkv written once (the bias table and
    its gradient are a few KB).  FLOPs: five contractions of N x N x head_dim
    per window and head (S, dP, dV, dK, dQ) over the unpadded N."""
    T = B * H * W
    C = heads * head_dim
    N = window * window
    return 7 * C * T * elem, 10 * N * C * T


def bwd_kernel_name(B: int, H: int, W: int, heads: int, window: int, cus: int) -> str:
    """Name of the backward kernel the library launches.  Mirrors its plan:
    head pairs for windows of 4 tiles with an even head count, unless their
    grid would leave CUs idle (runs of at least 8 windows per workgroup, two
    8-wave pair workgroups per CU), else one head per workgroup."""
    q = (window + 3) // 4
    hp = 1
    if q * q == 4 and heads % 2 == 0:
        groups = heads // 2
        windows = B * (H // window) * (W // window)
        runs = min(2 * cus // groups, windows, windows // 8)
        runs = max(runs, 1)
        if runs >= 8:
            runs -= runs % 8
        if runs * groups >= cus:
            hp = 2
    return f"wattn_bwd_bf16_kernel<{window}, {hp}>"


def fwd_kernel_name(window: int, heads: int, i8: bool = False) -> str:
    """Name of the bf16 (int8) forward kernel the library launches.  Mirrors
    its dispatch: head groups of 2, else 3, else 1 for windows of up to 4
    tiles of 16 tokens (window <= 8), 1 beyond."""
    q = (window + 3) // 4
    if q * q > 4:
        hg = 1
    else:
        hg = 2 if heads % 2 == 0 else 3 if heads % 3 == 0 else 1
    return f"wattn_fwd_persistent<{window}, {hg}, {'true' if i8 else 'false'}>"


def measured_traffic(workload: str, family: str = "wattn_fwd_bf16"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{family}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(family):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(name: str, sample_batch: int, min_seconds: float = 10.0, max_reps: int = 50,
                 gpu_out=None):
    """The fp64 oracle on the first `sample_batch` images of the workload, on
    every host core, repeated until about `min_seconds` of wall time; reported
    in the metric's unit (GB/s of algorithmic bytes).  With `gpu_out` (the
    library's output for the same images and the workload's first shift, as
    float64) the oracle's output is also compared with it, element by
    element, against the bf16 bars (max-abs 2e-2, mean-abs 2e-3)."""
    import oracle
    import synth
    w = synth.WORKLOADS[name]
    qkv, table = synth.workload_inputs(name, batch=sample_batch)
    reps, used, ref = 0, 0, None
    t0 = time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        ref, used = oracle.swin_wattn_fwd(qkv, table, w["window"], w["shifts"][0], return_threads=True)
        reps += 1
    dt = time.perf_counter() - t0
    nbytes, _ = algorithmic(sample_batch, w["H"], w["W"], w["heads"], w["head_dim"], w["window"])
    res = {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": used,
           "kind": "oracle",
           "sample": f"{name}, first {sample_batch} of {w['B']} images, whole forward x{reps} "
                     f"({dt:.1f} s wall, fp64, {used} threads)"}
    if gpu_out is not None:
        res["parity"] = _parity(gpu_out, ref)
    return res


def _parity(got, ref):
    """Element-by-element comparison of the library's bf16 forward output with
    the oracle's, against the bf16 bars (max-abs 2e-2, mean-abs 2e-3)."""
    err = abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    return {"max_abs": mx, "mean_abs": mean, "bar_max_abs": 2e-2, "bar_mean_abs": 2e-3,
            "elements": int(err.size), "ok": bool(mx <= 2e-2 and mean <= 2e-3)}


def i8_cpu_baseline(name: str, sample_batch: int, min_seconds: float = 10.0, max_reps: int = 50,
                    gpu_out=None):
    """The fp64 oracle (dequantize, then the forward) on the first
    `sample_batch` images of an INT8 workload, as cpu_baseline does (with
    `gpu_out`, the same comparison and bars)."""
    import oracle
    import synth
    a = synth.WORKLOADS[synth.I8_WORKLOADS[name]["attn"]]
    codes, scales, table = synth.i8_inputs(name, batch=sample_batch)
    reps, used, ref = 0, 0, None
    t0 = time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        ref, used = oracle.swin_wattn_fwd_i8(codes, scales, table, a["window"], a["shifts"][0],
                                             return_threads=True)
        reps += 1
    dt = time.perf_counter() - t0
    nbytes, _ = algorithmic(sample_batch, a["H"], a["W"], a["heads"], a["head_dim"], a["window"],
                            elem=1, out_elem=2)
    res = {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": used,
           "kind": "oracle",
           "sample": f"{name}, first {sample_batch} of {a['B']} images, whole forward x{reps} "
                     f"({dt:.1f} s wall, fp64, {used} threads)"}
    if gpu_out is not None:
        res["parity"] = _parity(gpu_out, ref)
    return res


def bwd_cpu_baseline(name: str, sample_batch: int, min_seconds: float = 10.0, max_reps: int = 50,
                     gpu_dqkv=None):
    """The fp64 oracle backward on the first `sample_batch` images, as
    cpu_baseline does for the forward.  With `gpu_dqkv` (the library's dq,
    dk, dv of the same images, float64) they are compared element by element
    against the backward's bars, per part: max error <= 2^-6 max |ref| and
    mean error <= 2^-8 mean |ref| (the table gradient sums over the whole
    batch and is not compared on a sample)."""
    import oracle
    import synth
    w = synth.WORKLOADS[name]
    qkv, table = synth.workload_inputs(name, batch=sample_batch)
    C = w["heads"] * w["head_dim"]
    n = sample_batch * w["H"] * w["W"] * C
    dout = synth.bf16_bits(synth.normal(synth.stream_key(w["seed"], 7), n, 1.0))
    dout = dout.reshape(sample_batch, w["H"], w["W"], C)
    reps, cores, ref = 0, 0, None
    t0 = time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        ref, _, cores = oracle.swin_wattn_bwd(qkv, table, dout, w["window"], w["shifts"][0],
                                              return_threads=True)
        reps += 1
    dt = time.perf_counter() - t0
    nbytes, _ = bwd_algorithmic(sample_batch, w["H"], w["W"], w["heads"], w["head_dim"], w["window"])
    res = {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
           "kind": "oracle",
           "sample": f"{name}, first {sample_batch} of {w['B']} images, whole backward x{reps} "
                     f"({dt:.1f} s wall, fp64, {cores} threads)"}
    if gpu_dqkv is not None:
        err = abs(gpu_dqkv - ref)
        worst_max = worst_mean = 0.0
        for part in range(3):  # dq, dk, dv
            e, r = err[:, :, :, part], abs(ref[:, :, :, part])
            worst_max = max(worst_max, float(e.max()) / (2.0 ** -6 * float(r.max()) + 1e-6))
            worst_mean = max(worst_mean, float(e.mean()) / (2.0 ** -8 * float(r.mean()) + 1e-7))
        res["parity"] = {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
                         "worst_max_over_bar": round(worst_max, 4),
                         "worst_mean_over_bar": round(worst_mean, 4), "elements": int(err.size),
                         "ok": bool(worst_max <= 1.0 and worst_mean <= 1.0)}
    return res


def time_steps(torch, step, K: int, warmup: int, stream, launches_per_step: int):
    """W untimed steps, then K timed steps between two synchronisations (HIP
    events on the launch stream); then K steps with an event pair around
    each.  Returns (total_ms, avg_launch_s, isolated_launch_s)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    # average launch duration: the HIP events around the timed region, on the
    # stream the kernel is launched on, over its launches (back to back: this
    # is what a kernel trace's mean duration agrees with)
    avg_launch_s = total_ms / 1e3 / (K * launches_per_step)
    # for reference, launches timed one by one (each event pair adds its own
    # overhead to the launch it brackets)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    isolated_s = sum(a.elapsed_time(b) for a, b in ev) / K / 1e3 / launches_per_step
    return total_ms, avg_launch_s, isolated_s


def linear_algorithmic(T, K, N, residual, elem=2):
    """Bytes: x read once, y written once, the residual read once.  FLOPs:
    one multiply-add per (token, input, output); a fused layer norm adds no
    bytes and is not counted as FLOPs."""
    return (T * K + T * N * (2 if residual else 1)) * elem, 2 * T * K * N


def linear_kernel_name(K: int, N: int, residual: bool, layernorm: bool = False) -> str:
    """The linear kernel the library launches (mirrors its dispatch: mode 0
    plain, 1 residual, 2 layer norm; 6, 4, 3 or 2 waves, the first that
    divides N / 32)."""
    ncb = N // 32
    waves = 6 if ncb % 6 == 0 else 4 if ncb % 4 == 0 else 3 if ncb % 3 == 0 else 2
    mode = 2 if layernorm else 1 if residual else 0
    return f"linear_fwd_kernel<{K // 32}, {mode}, {waves}>"


def linear_i8_kernel_name(K: int, N: int, residual: bool, out_i8: bool) -> str:
    """The INT8 linear kernel the library launches: k-steps of 64 channels,
    mode 3 bf16 output, 4 bf16 output + residual, 5 INT8 output; 9, 6, 4, 3 or
    2 waves, the first that divides N / 32)."""
    ncb = N // 32
    waves = (9 if ncb % 9 == 0 else 6 if ncb % 6 == 0 else 4 if ncb % 4 == 0 else
             3 if ncb % 3 == 0 else 2)
    mode = 5 if out_i8 else 4 if residual else 3
    return f"linear_fwd_kernel<{(K + 63) // 64}, {mode}, {waves}>"


def linear_i8_algorithmic(T, K, N, residual, out_i8):
    """Bytes: x (int8) read once, y (int8 or bf16) written once, the bf16
    residual read once.  FLOPs: one multiply-add per (token, input, output)."""
    return T * K + T * N * (1 if out_i8 else 2) + (T * N * 2 if residual else 0), 2 * T * K * N


def linear_i8_cpu_baseline(name: str, min_seconds: float = 10.0, gpu_rows=None):
    """The fp64 oracle of the INT8 linear layer on the first tokens of the
    workload (grown until one call takes about `min_seconds` / 4).  With
    `gpu_rows` (n -> the library's first n output rows) the outputs are
    compared: INT8 codes must be equal (both sides decide them by the same
    fp32 operations); bf16 output against |y - ref| <= 2^-7 |ref| + 2^-20
    (sum_c |x_c w_jc| x_scale w_scale_j + |b_j| + |r_j|)."""
    import numpy as np
    import oracle
    import synth
    w = synth.LINEAR_I8_WORKLOADS[name]
    n = 512
    while True:
        x, sx, wq, sw, b, r, so = synth.linear_i8_inputs(name, tokens=n)
        t0 = time.perf_counter()
        (_, ref, codes), used = oracle.linear_i8(x, sx, wq, sw, b, residual=r, so=so, return_threads=True)
        dt = time.perf_counter() - t0
        if dt >= min_seconds / 4 or n >= w["tokens"]:
            break
        n = min(w["tokens"], n * 4)
    reps = 1
    while time.perf_counter() - t0 < min_seconds and reps < 50:
        oracle.linear_i8(x, sx, wq, sw, b, residual=r, so=so)
        reps += 1
    dt = time.perf_counter() - t0
    nbytes, _ = linear_i8_algorithmic(n, w["K"], w["N"], w["residual"], w["out_i8"])
    res = {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": used,
           "kind": "oracle",
           "sample": f"{name}, first {n} of {w['tokens']} tokens x{reps} ({dt:.1f} s wall, "
                     f"exact integer sums + fp64, {used} threads)"}
    if gpu_rows is not None:
        got = gpu_rows(n)
        if w["out_i8"]:
            diff = int(np.count_nonzero(got != codes))
            res["parity"] = {"codes_differing": diff, "elements": int(codes.size), "ok": diff == 0}
        else:
            mag = ((np.abs(x.astype(np.float64)) @ np.abs(wq.astype(np.float64)).T) * (float(sx) * sw)
                   + np.abs(b.astype(np.float64)))
            if r is not None:
                mag = mag + np.abs(synth.bf16_to_f32(r).astype(np.float64))
            res["parity"] = _bound_parity(got, ref, mag * 2.0 ** -20)
    return res


def linear_i8_bench(args, torch, np) -> int:
    """One swin_linear_i8_fwd per step over a whole INT8 linear workload."""
    import shifted_window_attention_swin_amd as swa
    import synth
    w = synth.LINEAR_I8_WORKLOADS[args.workload]
    T, K, N, res, out_i8 = w["tokens"], w["K"], w["N"], w["residual"], w["out_i8"]
    dev = torch.device("cuda:0")
    x_np, sx, w_np, sw_np, b_np, r_np, so_np = synth.linear_i8_inputs(args.workload)
    x0 = torch.from_numpy(x_np).to(dev)
    wq = torch.from_numpy(w_np).to(dev)
    f32 = lambda a: None if a is None else torch.from_numpy(a).to(dev)
    sw, bias, so = f32(sw_np), f32(b_np), f32(so_np)
    r0 = torch.from_numpy(r_np.view(np.int16)).view(torch.bfloat16).to(dev) if res else None
    del x_np, r_np
    packed = torch.empty(N * ((K + 63) // 64) * 64, dtype=torch.int8, device=dev)
    swa.check(swa.swin_linear_i8_pack_weight(wq, packed, N, K), "pack_i8")
    nbytes, nflops = linear_i8_algorithmic(T, K, N, res, out_i8)
    sets = 1 if args.hot else 2 * MALL_BYTES // nbytes + 1
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    rs = [r0] + [r0.clone() for _ in range(sets - 1)] if res else [None] * sets
    ydt = torch.int8 if out_i8 else torch.bfloat16
    ys = [torch.empty(T, N, dtype=ydt, device=dev) for _ in range(sets)]
    stream = torch.cuda.current_stream()

    def step(i):
        k = i % sets
        swa.check(swa.swin_linear_i8_fwd(xs[k], float(sx), packed, sw, bias, rs[k], so, ys[k], T, K, N,
                                         stream), "linear_i8")

    K_ = args.steps
    total_ms, avg_launch_s, isolated_s = time_steps(torch, step, K_, args.warmup, stream, 1)
    value = nbytes * K_ / (total_ms / 1e3) / 1e9
    achieved = nbytes / avg_launch_s / 1e9
    result = {
        "metric": f"INT8 linear layer GB/s ({w['desc']}); % HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K_, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded SplitMix64/Box-Muller, int8 codes = rint(N(0, 32)) clipped to "
                "+-127; x scale 1/32, weight row scales 0.02/32 x (1 + 0.1 z), bias ~ N(0,0.02)"
                + (", output scales per q/k/v part" if out_i8 else ", bf16 residual ~ N(0,1)") + ")",
        "config": {"workload": args.workload, "desc": w["desc"], "tokens": T, "K": K, "N": N,
                   "residual": res, "out_dtype": "i8" if out_i8 else "bf16", "buffer_sets": sets,
                   "cache": "hot" if args.hot else "cold"},
        "tops": round(nflops * K_ / (total_ms / 1e3) / 1e12, 3),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, "linear_fwd"),
                     "kernel": linear_i8_kernel_name(K, N, res, out_i8),
                     "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "isolated_launch_us": round(isolated_s * 1e6, 3),
                     "alg_bytes_per_launch": nbytes, "alg_ops_per_launch": nflops,
                     "mfma_tops": round(nflops / avg_launch_s / 1e12, 3),
                     "mfma_peak_tops": INT8_PEAK_TOPS},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        step(0)  # one more launch (untimed) on the first buffer set, compared with the oracle
        torch.cuda.synchronize()
        result["cpu_baseline"] = linear_i8_cpu_baseline(
            args.workload, gpu_rows=lambda n: (lambda t: t.cpu().numpy() if t.dtype == torch.int8 else
                        t.float().cpu().numpy().astype(np.float64))(ys[0][:n]))
    print(json.dumps(result), flush=True)
    return 0


def _linear_workload(name: str):
    """(spec, layer norm?) of a linear or layer norm + linear workload."""
    import synth
    if name in synth.LN_LINEAR_WORKLOADS:
        return dict(synth.LN_LINEAR_WORKLOADS[name], residual=False), True
    return synth.LINEAR_WORKLOADS[name], False


def linear_cpu_baseline(name: str, min_seconds: float = 10.0, gpu_rows=None):
    """The fp64 oracle on the first tokens of the workload (grown until one
    call takes about `min_seconds`), reported in GB/s of algorithmic bytes.
    With `gpu_rows` (n -> the library's first n output rows, float64) the
    oracle's rows are compared with them element by element against the
    linear layer's bound: |y - ref| <= 2^-7 |ref| + 2^-20 (sum_c |x_c w_jc|
    + |b_j| + |r_j|); with the layer norm, 2^-7 |ref| + 2^-7 sum_c (|xn_c| +
    |beta_c|) |w_jc| + 2^-20 |b_j| (gamma o W rounded to bf16)."""
    import numpy as np
    import oracle
    import synth
    w, ln = _linear_workload(name)

    def run(n):
        if ln:
            x, g, be, wt, b = synth.ln_linear_inputs(name, tokens=n)
            return (lambda: oracle.linear(oracle.layernorm(x, g, be), wt, b, return_threads=True),
                    (x, g, be, wt, b))
        x, wt, b, r = synth.linear_inputs(name, tokens=n)
        return lambda: oracle.linear(x, wt, b, r, return_threads=True), (x, wt, b, r)

    n = 512
    while True:
        call, inputs = run(n)
        t0 = time.perf_counter()
        ref, used = call()
        dt = time.perf_counter() - t0
        if dt >= min_seconds / 4 or n >= w["tokens"]:
            break
        n = min(w["tokens"], n * 4)
    reps = 1
    while time.perf_counter() - t0 < min_seconds and reps < 50:
        call()
        reps += 1
    dt = time.perf_counter() - t0
    nbytes, _ = linear_algorithmic(n, w["K"], w["N"], w["residual"])
    res = {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": used,
           "kind": "oracle",
           "sample": f"{name}, first {n} of {w['tokens']} tokens x{reps} ({dt:.1f} s wall, fp64, "
                     f"{used} threads)"}
    if gpu_rows is not None:
        got = gpu_rows(n)
        f64 = lambda bits: synth.bf16_to_f32(bits).astype(np.float64)
        if ln:
            x, g, be, wt, b = inputs
            xn = oracle.layernorm(x, g, be)
            extra = ((np.abs(xn) + np.abs(be.astype(np.float64))) @ np.abs(f64(wt)).T * 2.0 ** -7
                     + np.abs(b.astype(np.float64)) * 2.0 ** -20)
        else:
            x, wt, b, r = inputs
            mag = np.abs(f64(x)) @ np.abs(f64(wt)).T + np.abs(b.astype(np.float64))
            if r is not None:
                mag = mag + np.abs(f64(r))
            extra = mag * 2.0 ** -20
        res["parity"] = _bound_parity(got, ref, extra)
    return res


def _bound_parity(got, ref, extra):
    """Element-by-element comparison against the per-element bound
    2^-7 |ref| + extra: the worst ratio of error to bound, <= 1 passes."""
    err = abs(got - ref)
    worst = float((err / (2.0 ** -7 * abs(ref) + extra)).max())
    return {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
            "worst_err_over_bound": round(worst, 4), "elements": int(err.size), "ok": bool(worst <= 1.0)}


def linear_bench(args, torch, np) -> int:
    """One swin_linear_fwd per step over a whole linear workload."""
    import shifted_window_attention_swin_amd as swa
    import synth
    w, ln = _linear_workload(args.workload)
    T, K, N, res = w["tokens"], w["K"], w["N"], w["residual"]
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    if ln:
        x_np, g_np, be_np, w_np, b_np = synth.ln_linear_inputs(args.workload)
        gamma, beta = torch.from_numpy(g_np).to(dev), torch.from_numpy(be_np).to(dev)
        r_np = None
    else:
        x_np, w_np, b_np, r_np = synth.linear_inputs(args.workload)
    x0, wt, bias = bf(x_np), bf(w_np), torch.from_numpy(b_np).to(dev)
    r0 = bf(r_np) if res else None
    del x_np, r_np
    packed = torch.empty_like(wt)
    if ln:
        consts = torch.empty(2, N, dtype=torch.float32, device=dev)
        swa.check(swa.swin_ln_linear_pack_weight(wt, gamma, beta, bias, packed, consts, N, K), "pack")
    else:
        swa.check(swa.swin_linear_pack_weight(wt, packed, N, K), "pack")
    nbytes, nflops = linear_algorithmic(T, K, N, res)
    sets = 1 if args.hot else 2 * MALL_BYTES // nbytes + 1
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    rs = [r0] + [r0.clone() for _ in range(sets - 1)] if res else [None] * sets
    ys = [torch.empty(T, N, dtype=torch.bfloat16, device=dev) for _ in range(sets)]
    stream = torch.cuda.current_stream()

    def step(i):
        k = i % sets
        if ln:
            swa.check(swa.swin_ln_linear_fwd(xs[k], packed, consts, 1e-5, ys[k], T, K, N, stream),
                      "ln_linear")
        else:
            swa.check(swa.swin_linear_fwd(xs[k], packed, bias, rs[k], ys[k], T, K, N, stream), "linear")

    K_ = args.steps
    total_ms, avg_launch_s, isolated_s = time_steps(torch, step, K_, args.warmup, stream, 1)
    value = nbytes * K_ / (total_ms / 1e3) / 1e9
    achieved = nbytes / avg_launch_s / 1e9
    result = {
        "metric": f"{'layer norm + ' if ln else ''}linear layer GB/s ({w['desc']}, bf16); % HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K_, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller, " + ("x ~ N(0.5,2), gamma ~ N(1,0.1), "
                                                                "beta ~ N(0,0.1)" if ln else "x ~ N(0,1)")
                + ", W and bias ~ N(0,0.02))",
        "config": {"workload": args.workload, "desc": w["desc"], "tokens": T, "K": K, "N": N,
                   "residual": res, "layernorm": ln, "buffer_sets": sets,
                   "cache": "hot" if args.hot else "cold"},
        "tflops": round(nflops * K_ / (total_ms / 1e3) / 1e12, 3),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, "linear_fwd"),
                     "kernel": linear_kernel_name(K, N, res, ln),
                     "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "isolated_launch_us": round(isolated_s * 1e6, 3),
                     "alg_bytes_per_launch": nbytes, "alg_flops_per_launch": nflops,
                     "mfma_tflops": round(nflops / avg_launch_s / 1e12, 3),
                     "mfma_peak_tflops": BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        step(0)  # one more launch (untimed) on the first buffer set, compared with the oracle
        torch.cuda.synchronize()
        result["cpu_baseline"] = linear_cpu_baseline(
            args.workload, gpu_rows=lambda n: (lambda t: t.cpu().numpy() if t.dtype == torch.int8 else
                        t.float().cpu().numpy().astype(np.float64))(ys[0][:n]))
    print(json.dumps(result), flush=True)
    return 0


def ln_attn_algorithmic(B, H, W, heads, head_dim, window):
    """Bytes: x read once + out written once.  FLOPs: the QKV projection
    (2 C 3C per token) and the attention's two contractions over the
    unpadded window (4 N C per token)."""
    T = B * H * W
    C = heads * head_dim
    return 4 * C * T, 2 * T * C * 3 * C + 4 * window * window * C * T


def ln_attn_cpu_baseline(name: str, min_seconds: float = 10.0, max_reps: int = 50, gpu_out=None):
    """The fp64 oracle chain (layer norm, linear, attention) on the first
    images of the workload, repeated for about `min_seconds`.  With `gpu_out`
    (the library's output of those images, float64) compared as
    cpu_baseline does."""
    import oracle
    import synth
    spec = synth.LN_ATTN_WORKLOADS[name]
    a = synth.WORKLOADS[spec["attn"]]
    M, s = a["window"], a["shifts"][0]
    nb = 2
    x, g, be, w, b, t = synth.ln_attn_inputs(name, batch=nb)
    B, H, W, C = x.shape
    reps, cores, ref = 0, 0, None
    t0 = time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        xn = oracle.layernorm(x, g, be)
        qkv, cores = oracle.linear(xn, w, b, return_threads=True)
        ref = oracle.swin_wattn_fwd(qkv.reshape(B, H, W, 3, C // 32, 32), t, M, s)
        reps += 1
    dt = time.perf_counter() - t0
    nbytes, _ = ln_attn_algorithmic(nb, H, W, C // 32, 32, M)
    res = {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
           "kind": "oracle",
           "sample": f"{name}, first {nb} of {a['B']} images, layer norm + linear + attention "
                     f"x{reps} ({dt:.1f} s wall, fp64, {cores} threads)"}
    if gpu_out is not None:
        res["parity"] = _parity(gpu_out[:nb], ref)
    return res


def ln_attn_bench(args, torch, np) -> int:
    """One swin_ln_qkv_wattn_fwd per step over the whole workload; the
    two-kernel chain (swin_ln_linear_fwd, then swin_wattn_fwd) is timed
    beside it on the same buffers."""
    import shifted_window_attention_swin_amd as swa
    import synth
    spec = synth.LN_ATTN_WORKLOADS[args.workload]
    a = synth.WORKLOADS[spec["attn"]]
    B, H, W, nh, d, M = a["B"], a["H"], a["W"], a["heads"], a["head_dim"], a["window"]
    s = a["shifts"][0]
    C = nh * d
    T = B * H * W
    dev = torch.device("cuda:0")
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev)
    x_np, g_np, be_np, w_np, b_np, t_np = synth.ln_attn_inputs(args.workload)
    x0, wd = bf(x_np), bf(w_np)
    del x_np
    packed = torch.empty_like(wd)
    consts = torch.empty(2, 3 * C, dtype=torch.float32, device=dev)
    swa.check(swa.swin_ln_linear_pack_weight(wd, torch.from_numpy(g_np).to(dev),
                                             torch.from_numpy(be_np).to(dev),
                                             torch.from_numpy(b_np).to(dev), packed, consts,
                                             3 * C, C), "pack")
    table = torch.from_numpy(t_np).to(dev)
    nbytes, nflops = ln_attn_algorithmic(B, H, W, nh, d, M)
    sets = 1 if args.hot else 2 * MALL_BYTES // nbytes + 1
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    outs = [torch.empty(B, H, W, C, dtype=torch.bfloat16, device=dev) for _ in range(sets)]
    stream = torch.cuda.current_stream()

    def step(i):
        k = i % sets
        swa.check(swa.swin_ln_qkv_wattn_fwd(xs[k], packed, consts, 1e-5, table, outs[k], B, H, W,
                                            nh, d, M, s, stream), "ln_qkv_wattn")

    K = args.steps
    total_ms, avg_launch_s, isolated_s = time_steps(torch, step, K, args.warmup, stream, 1)
    # the two-kernel chain on the same inputs: the layer norm + QKV
    # projection writes qkv, the attention reads it
    qkv = torch.empty(T, 3 * C, dtype=torch.bfloat16, device=dev)

    def chain(i):
        k = i % sets
        swa.check(swa.swin_ln_linear_fwd(xs[k], packed, consts, 1e-5, qkv, T, C, 3 * C, stream),
                  "ln_linear")
        swa.check(swa.swin_wattn_fwd(qkv, table, outs[k], B, H, W, nh, d, M, s, stream), "fwd")

    chain_ms, _, _ = time_steps(torch, chain, K, args.warmup, stream, 1)
    value = nbytes * K / (total_ms / 1e3) / 1e9
    tflops = nflops / avg_launch_s / 1e12
    mfma_bound = nflops / nbytes > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 3), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    else:
        ach = nbytes / avg_launch_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": measured_traffic(args.workload, "ln_qkv_wattn"),
                 "kernel": f"ln_qkv_wattn_kernel<{M}, {C // 32}>",
                 "avg_launch_us": round(avg_launch_s * 1e6, 3),
                 "isolated_launch_us": round(isolated_s * 1e6, 3),
                 "alg_bytes_per_launch": nbytes, "alg_flops_per_launch": nflops,
                 "hbm_gbs": round(nbytes / avg_launch_s / 1e9, 2),
                 "flop_per_byte": round(nflops / nbytes, 1)})
    result = {
        "metric": f"layer norm + QKV + window attention GB/s & TFLOP/s ({spec['desc']}, bf16)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller, x ~ N(0.5,2), gamma ~ N(1,0.1), "
                "beta ~ N(0,0.1), W and bias ~ N(0,0.02), bias table ~ N(0,0.02))",
        "config": {"workload": args.workload, "desc": spec["desc"], "B": B, "H": H, "W": W,
                   "heads": nh, "head_dim": d, "window": M, "shift": s, "buffer_sets": sets,
                   "cache": "hot" if args.hot else "cold"},
        "tflops": round(nflops * K / (total_ms / 1e3) / 1e12, 3),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "two_kernel_chain_us": round(chain_ms / K * 1e3, 3),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        step(0)  # one more launch (untimed) of the fused call, compared with the oracle chain
        torch.cuda.synchronize()
        result["cpu_baseline"] = ln_attn_cpu_baseline(
            args.workload, gpu_out=outs[0][:2].float().cpu().numpy().astype(np.float64))
    print(json.dumps(result), flush=True)
    return 0


def bwd_bench(args, torch, np) -> int:
    """One swin_wattn_bwd per step over the whole workload (first shift)."""
    import shifted_window_attention_swin_amd as swa
    import synth
    w = synth.WORKLOADS[args.workload]
    B, H, W, nh, d, M = w["B"], w["H"], w["W"], w["heads"], w["head_dim"], w["window"]
    s = w["shifts"][0]
    C = nh * d
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    qkv_np, table_np = synth.workload_inputs(args.workload)
    q0, table = bf(qkv_np), torch.from_numpy(table_np).to(dev)
    del qkv_np
    g0 = bf(synth.bf16_bits(synth.normal(synth.stream_key(w["seed"], 7), B * H * W * C, 1.0)))
    nbytes, nflops = bwd_algorithmic(B, H, W, nh, d, M)
    sets = 1 if args.hot else 2 * MALL_BYTES // nbytes + 1
    qs = [q0] + [q0.clone() for _ in range(sets - 1)]
    gs = [g0] + [g0.clone() for _ in range(sets - 1)]
    dqs = [torch.empty_like(q0) for _ in range(sets)]
    dt = torch.empty_like(table)
    stream = torch.cuda.current_stream()

    def step(i):
        k = i % sets
        swa.check(swa.swin_wattn_bwd(qs[k], table, gs[k], dqs[k], dt, B, H, W, nh, d, M, s, stream),
                  "bwd")

    K = args.steps
    total_ms, avg_launch_s, isolated_s = time_steps(torch, step, K, args.warmup, stream, 1)
    value = nbytes * K / (total_ms / 1e3) / 1e9
    achieved = nbytes / avg_launch_s / 1e9
    result = {
        "metric": f"shifted-window attn bwd GB/s ({w['desc']}, bf16); % HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller, qkv and dout ~ N(0,1), bias table ~ N(0,0.02))",
        "config": {"workload": args.workload, "pass": "backward", "desc": w["desc"], "B": B, "H": H,
                   "W": W, "heads": nh, "head_dim": d, "window": M, "shift": s,
                   "buffer_sets": sets, "cache": "hot" if args.hot else "cold"},
        "tflops": round(nflops * K / (total_ms / 1e3) / 1e12, 3),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        # a step is two launches (the bias-gradient zero fill, then the
        # backward kernel); the per-step time is charged to the backward kernel
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, "wattn_bwd_bf16"),
                     "kernel": bwd_kernel_name(B, H, W, nh, M,
                                               torch.cuda.get_device_properties(0).multi_processor_count),
                     "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "isolated_launch_us": round(isolated_s * 1e6, 3),
                     "alg_bytes_per_launch": nbytes, "alg_flops_per_launch": nflops,
                     "mfma_tflops": round(nflops / avg_launch_s / 1e12, 3),
                     "mfma_peak_tflops": BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        # one more launch (untimed): its dq, dk, dv of the sampled images are
        # compared with the oracle's
        sb = min(args.cpu_sample_batch, B, 8)
        swa.check(swa.swin_wattn_bwd(qs[0], table, gs[0], dqs[0], dt, B, H, W, nh, d, M, s, stream), "bwd")
        torch.cuda.synchronize()
        got = dqs[0][:sb].float().cpu().numpy().astype(np.float64).reshape(sb, H, W, 3, nh, d)
        result["cpu_baseline"] = bwd_cpu_baseline(args.workload, sb, gpu_dqkv=got)
    print(json.dumps(result), flush=True)
    return 0


def i8_bench(args, torch, np) -> int:
    """One swin_wattn_fwd_i8 per step over the whole INT8 workload (first
    shift)."""
    import shifted_window_attention_swin_amd as swa
    import synth
    spec = synth.I8_WORKLOADS[args.workload]
    a = synth.WORKLOADS[spec["attn"]]
    B, H, W, nh, d, M = a["B"], a["H"], a["W"], a["heads"], a["head_dim"], a["window"]
    s = a["shifts"][0]
    dev = torch.device("cuda:0")
    codes, scales, table_np = synth.i8_inputs(args.workload)
    q0 = torch.from_numpy(codes).to(dev)
    table = torch.from_numpy(table_np).to(dev)
    del codes
    sq, sk, sv = (float(x) for x in scales)
    nbytes, nflops = algorithmic(B, H, W, nh, d, M, elem=1, out_elem=2)
    sets = 1 if args.hot else 2 * MALL_BYTES // nbytes + 1
    qs = [q0] + [q0.clone() for _ in range(sets - 1)]
    outs = [torch.empty(B, H, W, nh * d, dtype=torch.bfloat16, device=dev) for _ in range(sets)]
    stream = torch.cuda.current_stream()

    def step(i):
        k = i % sets
        swa.check(swa.swin_wattn_fwd_i8(qs[k], sq, sk, sv, 0.0, table, outs[k], B, H, W, nh, d, M, s,
                                        stream), "fwd_i8")

    K = args.steps
    total_ms, avg_launch_s, isolated_s = time_steps(torch, step, K, args.warmup, stream, 1)
    value = nbytes * K / (total_ms / 1e3) / 1e9
    achieved = nbytes / avg_launch_s / 1e9
    result = {
        "metric": f"shifted-window attn fwd GB/s & TFLOP/s ({spec['desc']}); % HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # int8 codes in; exact products and sums on the bf16 MFMA path, bf16 out
        "dtype": "i8",
        "data": "synthetic (seeded SplitMix64/Box-Muller, int8 codes = rint(N(0, 32)) clipped to "
                "+-127, scales (q, k, v) = " + ", ".join(f"{x:g}" for x in scales)
                + ", bias table ~ N(0,0.02))",
        "config": {"workload": args.workload, "desc": spec["desc"], "B": B, "H": H, "W": W,
                   "heads": nh, "head_dim": d, "window": M, "shift": s, "buffer_sets": sets,
                   "cache": "hot" if args.hot else "cold", "out_dtype": "bf16"},
        "tflops": round(nflops * K / (total_ms / 1e3) / 1e12, 3),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, "wattn_fwd_i8"),
                     "kernel": fwd_kernel_name(M, nh, i8=True),
                     "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "isolated_launch_us": round(isolated_s * 1e6, 3),
                     "alg_bytes_per_launch": nbytes, "alg_flops_per_launch": nflops,
                     "mfma_tflops": round(nflops / avg_launch_s / 1e12, 3),
                     "mfma_peak_tflops": BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        # one more launch (untimed): its output on the sampled images is
        # compared with the oracle's
        sb = min(args.cpu_sample_batch, B)
        swa.check(swa.swin_wattn_fwd_i8(qs[0], sq, sk, sv, 0.0, table, outs[0], B, H, W, nh, d, M, s,
                                        stream), "fwd_i8")
        torch.cuda.synchronize()
        got = outs[0][:sb].float().cpu().numpy().astype(np.float64)
        result["cpu_baseline"] = i8_cpu_baseline(args.workload, sb, gpu_out=got)
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # the GPU needs some tens of milliseconds of sustained load before its
    # launches reach steady speed: 1000 warmup launches are about 60 ms here
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="swin-l-s1")
    ap.add_argument("--backward", action="store_true", help="time the attention backward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-batch", type=int, default=64)
    ap.add_argument("--hot", action="store_true", help="one buffer set (working set may sit in cache)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run 4 plain device-to-device copies of BYTES bytes (calibrates the "
                         "HBM byte counters of a profiler) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; the forward shards by batch with no "
              "communication, so there is no multi-GPU run to make (--gpus must be 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_probe:
        n = args.copy_probe // 16 * 16
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda:0")
        dst = [torch.empty_like(src) for _ in range(2)]
        for i in range(4):
            dst[i % 2].copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 4}), flush=True)
        return 0

    import shifted_window_attention_swin_amd as swa
    import synth

    if args.workload in synth.LINEAR_WORKLOADS or args.workload in synth.LN_LINEAR_WORKLOADS:
        return linear_bench(args, torch, np)
    if args.workload in synth.LN_ATTN_WORKLOADS:
        return ln_attn_bench(args, torch, np)
    if args.workload in synth.I8_WORKLOADS:
        return i8_bench(args, torch, np)
    if args.workload in synth.LINEAR_I8_WORKLOADS:
        return linear_i8_bench(args, torch, np)
    if args.backward:
        return bwd_bench(args, torch, np)
    w = synth.WORKLOADS[args.workload]
    if w["dtype"] != "bf16":
        print("bench.py: the benchmark times the bf16 path", file=sys.stderr)
        return 2
    B, H, W, nh, d, M = w["B"], w["H"], w["W"], w["heads"], w["head_dim"], w["window"]
    shifts = w["shifts"]
    dev = torch.device("cuda:0")

    qkv_np, table_np = synth.workload_inputs(args.workload)
    q0 = torch.from_numpy(qkv_np.view(np.int16)).view(torch.bfloat16).to(dev)
    table = torch.from_numpy(table_np).to(dev)
    del qkv_np
    nbytes, nflops = algorithmic(B, H, W, nh, d, M)
    nbytes *= len(shifts)
    nflops *= len(shifts)
    footprint = nbytes // len(shifts)
    sets = 1 if args.hot else 2 * MALL_BYTES // footprint + 1  # sets * footprint > 2 x MALL
    qs = [q0] + [q0.clone() for _ in range(sets - 1)]
    outs = [torch.empty(B, H, W, nh * d, dtype=torch.bfloat16, device=dev) for _ in range(sets)]
    stream = torch.cuda.current_stream()

    def step(i):
        k = i % sets
        for s in shifts:
            swa.check(swa.swin_wattn_fwd(qs[k], table, outs[k], B, H, W, nh, d, M, s, stream), "fwd")

    K = args.steps
    total_ms, avg_launch_s, isolated_s = time_steps(torch, step, K, args.warmup, stream, len(shifts))
    ms_per_step = total_ms / K
    value = nbytes * K / (total_ms / 1e3) / 1e9
    achieved = (nbytes / len(shifts)) / avg_launch_s / 1e9
    traffic = measured_traffic(args.workload)
    result = {
        # the headline metric names Swin-L stage 1; other workloads say what they are
        "metric": METRIC if args.workload == "swin-l-s1" else
        f"shifted-window attn fwd GB/s & TFLOP/s ({w['desc']}, {w['dtype']}); % HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller, qkv ~ N(0,1), bias table ~ N(0,0.02))",
        "config": {"workload": args.workload, "desc": w["desc"], "B": B, "H": H, "W": W, "heads": nh,
                   "head_dim": d, "window": M, "shifts": list(shifts),
                   "buffer_sets": sets, "cache": "hot" if args.hot else "cold"},
        "tflops": round(nflops * K / (total_ms / 1e3) / 1e12, 3),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": fwd_kernel_name(M, nh),
                     "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "isolated_launch_us": round(isolated_s * 1e6, 3),
                     "alg_bytes_per_launch": nbytes // len(shifts),
                     "alg_flops_per_launch": nflops // len(shifts),
                     "mfma_tflops": round((nflops / len(shifts)) / avg_launch_s / 1e12, 3),
                     "mfma_peak_tflops": BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        # one more launch (untimed) with the workload's first shift: its
        # output on the sampled images is compared with the oracle's
        sb = min(args.cpu_sample_batch, B)
        swa.check(swa.swin_wattn_fwd(qs[0], table, outs[0], B, H, W, nh, d, M, shifts[0], stream), "fwd")
        torch.cuda.synchronize()
        got = outs[0][:sb].float().cpu().numpy().astype(np.float64)
        result["cpu_baseline"] = cpu_baseline(args.workload, sb, gpu_out=got)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
