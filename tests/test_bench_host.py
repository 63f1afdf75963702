"""Host logic of bench.py, on the CPU: the algorithmic byte and FLOP counts
the roofline divides by, the kernel names it reports (which mirror the
launchers' dispatch rules), the gating of committed traffic records by the
kernel source hash, and the one-GPU contract of --gpus."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _window_sum(B, H, W, heads, d, M):
    """FLOPs summed window by window: per (image, window, head) two N x N x d
    contractions (scores, then weights times values), 2 FLOPs per
    multiply-add."""
    N = M * M
    windows = B * (H // M) * (W // M)
    return windows * heads * 2 * (2 * N * N * d)


@pytest.mark.parametrize("B,H,W,heads,M,mb,gflop", [
    (32, 56, 56, 3, 7, 77.07, 1.888),     # Swin-T stage 1
    (64, 14, 14, 12, 7, 38.54, 0.944),    # Swin-T stage 3, one call
    (64, 56, 56, 6, 7, 308.28, 7.553),    # Swin-L stage 1
    (16, 96, 96, 6, 12, 226.49, 16.307),  # Swin-L at 384 px, window 12
])
def test_forward_algorithmic_counts(B, H, W, heads, M, mb, gflop):
    nbytes, flops = bench.algorithmic(B, H, W, heads, 32, M)
    T, C = B * H * W, heads * 32
    assert nbytes == T * 3 * C * 2 + T * C * 2  # qkv read once, out written once, bf16
    assert flops == _window_sum(B, H, W, heads, 32, M)
    assert round(nbytes / 1e6, 2) == mb and round(flops / 1e9, 3) == gflop


def test_forward_algorithmic_headline_exact():
    assert bench.algorithmic(64, 56, 56, 6, 32, 7) == (308281344, 7552892928)
    # int8 q, k, v codes, bf16 output: 3 C T + 2 C T bytes
    T, C = 64 * 56 * 56, 192
    assert bench.algorithmic(64, 56, 56, 6, 32, 7, elem=1, out_elem=2)[0] == 3 * C * T + 2 * C * T


def test_backward_algorithmic_counts():
    nbytes, flops = bench.bwd_algorithmic(64, 56, 56, 6, 32, 7)
    T, C = 64 * 56 * 56, 192
    assert nbytes == (3 * C + C + 3 * C) * T * 2 == 539492352  # qkv, dout read; dqkv written
    # five contractions per window and head: S, dP, dV, dK, dQ
    assert flops == _window_sum(64, 56, 56, 6, 32, 7) // 2 * 5


def test_linear_and_fused_counts():
    T = 64 * 56 * 56
    assert bench.linear_algorithmic(T, 192, 576, False) == ((T * 192 + T * 576) * 2, 2 * T * 192 * 576)
    assert bench.linear_algorithmic(T, 192, 192, True)[0] == (T * 192 + 2 * T * 192) * 2
    assert bench.linear_i8_algorithmic(T, 192, 576, False, True) == (T * 192 + T * 576, 2 * T * 192 * 576)
    assert bench.linear_i8_algorithmic(T, 192, 192, True, False)[0] == T * 192 + T * 192 * 2 + T * 192 * 2
    nbytes, flops = bench.ln_attn_algorithmic(64, 56, 56, 6, 32, 7)
    assert nbytes == 2 * T * 192 * 2  # x read, out written
    assert flops == 2 * T * 192 * 576 + _window_sum(64, 56, 56, 6, 32, 7)


@pytest.mark.parametrize("window,heads,i8,name", [
    (7, 6, False, "wattn_fwd_persistent<7, 2, false>"),   # even head count: pairs
    (7, 3, False, "wattn_fwd_persistent<7, 3, false>"),   # odd multiple of 3: triples
    (7, 5, False, "wattn_fwd_persistent<7, 1, false>"),
    (8, 9, True, "wattn_fwd_persistent<8, 3, true>"),
    (4, 6, False, "wattn_fwd_persistent<4, 2, false>"),   # one-tile windows group heads too
    (12, 6, False, "wattn_fwd_persistent<12, 1, false>"),  # 9-tile windows: one head
    (9, 4, True, "wattn_fwd_persistent<9, 1, true>"),
])
def test_forward_kernel_name(window, heads, i8, name):
    assert bench.fwd_kernel_name(window, heads, i8) == name


def test_backward_kernel_name():
    # Swin-L stage 1: 3 head pairs x 168 runs cover the 256 CUs -> pairs
    assert bench.bwd_kernel_name(64, 56, 56, 6, 7, 256) == "wattn_bwd_bf16_kernel<7, 2>"
    # Swin-T stage 3: 256 windows -> at most 32 runs of 8; 6 pairs x 32 = 192 < 256 -> one head
    assert bench.bwd_kernel_name(64, 14, 14, 12, 7, 256) == "wattn_bwd_bf16_kernel<7, 1>"
    # odd head count: no pairs
    assert bench.bwd_kernel_name(32, 56, 56, 3, 7, 256) == "wattn_bwd_bf16_kernel<7, 1>"
    # 9-tile windows: one head
    assert bench.bwd_kernel_name(16, 96, 96, 6, 12, 256) == "wattn_bwd_bf16_kernel<12, 1>"


def test_linear_kernel_names():
    assert bench.linear_kernel_name(192, 576, False) == "linear_fwd_kernel<6, 0, 6>"
    assert bench.linear_kernel_name(192, 192, True) == "linear_fwd_kernel<6, 1, 6>"
    assert bench.linear_kernel_name(192, 576, False, layernorm=True) == "linear_fwd_kernel<6, 2, 6>"
    assert bench.linear_kernel_name(96, 288, False) == "linear_fwd_kernel<3, 0, 3>"  # 9 blocks
    assert bench.linear_kernel_name(384, 1152, False) == "linear_fwd_kernel<12, 0, 6>"
    assert bench.linear_kernel_name(64, 64, True) == "linear_fwd_kernel<2, 1, 2>"
    assert bench.linear_i8_kernel_name(192, 576, False, True) == "linear_fwd_kernel<3, 5, 9>"
    assert bench.linear_i8_kernel_name(192, 192, True, False) == "linear_fwd_kernel<3, 4, 6>"
    assert bench.linear_i8_kernel_name(96, 288, False, True) == "linear_fwd_kernel<2, 5, 9>"


def test_traffic_record_gated_by_source_hash(monkeypatch):
    rec_path = os.path.join(ROOT, "profiles", "wattn_fwd_bf16_swin-l-s1_traffic.json")
    with open(rec_path) as f:
        rec = json.load(f)
    got = bench.measured_traffic("swin-l-s1")
    if rec["kernel_source_sha256_16"] == bench.kernel_source_hash("wattn_fwd_bf16"):
        assert got == rec["hbm_bytes_per_launch"]
        # within a few percent of the algorithmic bytes
        assert 0.99 < got / bench.algorithmic(64, 56, 56, 6, 32, 7)[0] < 1.10
    else:
        assert got is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda family="wattn_fwd_bf16": "0" * 16)
    assert bench.measured_traffic("swin-l-s1") is None
    assert bench.measured_traffic("no-such-workload") is None


def test_source_hash_covers_each_family():
    hashes = {fam: bench.kernel_source_hash(fam) for fam in bench.KERNEL_SOURCES}
    assert all(len(h) == 16 for h in hashes.values())
    # the bf16 and int8 forwards share their sources, the other families differ
    assert hashes["wattn_fwd_bf16"] == hashes["wattn_fwd_i8"]
    assert len(set(hashes.values())) == len(hashes) - 1


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                         env=dict(os.environ, **env), capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""


def test_reported_kernel_names_match_the_traces():
    # each committed rocprofv3 summary names, in its title, the kernel that
    # bench.py reported for the run, and lists the kernels the trace saw:
    # the mirrors of the dispatch rules must name a kernel that really ran
    import glob
    import re
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert len(paths) >= 10
    for path in paths:
        with open(path) as f:
            text = f.read()
        reported = re.search(r"rocprofv3 summary: (.+?), (backward of )?workload", text).group(1)
        traced = [re.sub(r"^void |swinattn::\(anonymous namespace\)::|\(swinattn::\w+\)$", "", n)
                  for n in re.findall(r"\| `([^`]+)` \|", text)]
        traced = [n.replace("swinattn::(anonymous namespace)::", "") for n in traced]
        assert reported in traced, (os.path.basename(path), reported, traced)
