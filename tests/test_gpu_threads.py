"""The library's calls from several host threads at once, each thread on a
stream of its own.

The header promises that swin_wattn_fwd and the linear calls may be called
concurrently: they allocate nothing, and the per-device launch caches
(occupancy of each kernel instantiation, compute-unit count) are filled
lazily with atomic stores.  The test runs in a fresh child process, so that
those caches start empty and the threads fill them concurrently: four
threads, released together, each run forwards of a different window and
head count (different kernel instantiations and launch plans) and a linear
layer, twenty times, on their own streams.  Their outputs must equal, bit
for bit, the same calls made one after another on one stream afterwards
(every call is deterministic), and the first thread's forward must match the
fp64 oracle within the bf16 bars.  The case prints its name before touching
the GPU."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import threading
import numpy as np
import torch
import oracle
import shifted_window_attention_swin_amd as swa
import synth

dev = torch.device("cuda:0")
bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
CASES = [(2, 20, 20, 3, 5, 2), (2, 24, 24, 5, 6, 3), (1, 30, 30, 2, 10, 4), (1, 22, 22, 7, 11, 5)]
REPS = 20
inputs = []
for i, (B, H, W, nh, M, s) in enumerate(CASES):
    qkv, table = synth.make_inputs(B, H, W, nh, 32, M, seed=300 + i, dtype="bf16")
    C = nh * 32
    x, w, b, _ = synth.make_linear_inputs(B * H * W, C, C, 310 + i, False)
    wd = bf(w)
    packed = torch.empty_like(wd)
    swa.check(swa.swin_linear_pack_weight(wd, packed, C, C), "pack")
    inputs.append((qkv, bf(qkv), torch.from_numpy(table).to(dev), bf(x), packed,
                   torch.from_numpy(b).to(dev)))
torch.cuda.synchronize()

def run(i, stream, outs):
    B, H, W, nh, M, s = CASES[i]
    _, q, t, x, packed, b = inputs[i]
    C = nh * 32
    for r in range(REPS):
        swa.check(swa.swin_wattn_fwd(q, t, outs[0][r], B, H, W, nh, 32, M, s, stream), "fwd")
        swa.check(swa.swin_linear_fwd(x, packed, b, None, outs[1][r], B * H * W, C, C, stream), "linear")

def buffers(i):
    B, H, W, nh, M, s = CASES[i]
    C = nh * 32
    return ([torch.full((B, H, W, C), float("nan"), dtype=torch.bfloat16, device=dev) for _ in range(REPS)],
            [torch.full((B * H * W, C), float("nan"), dtype=torch.bfloat16, device=dev) for _ in range(REPS)])

streams = [torch.cuda.Stream() for _ in CASES]  # default priority
par = [buffers(i) for i in range(len(CASES))]
torch.cuda.synchronize()
gate = threading.Barrier(len(CASES))
errors = []

def worker(i):
    try:
        gate.wait()
        run(i, streams[i], par[i])
        streams[i].synchronize()
    except Exception as e:  # reported by the main thread
        errors.append(repr(e))

threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
for th in threads:
    th.start()
for th in threads:
    th.join()
assert not errors, errors

seq = [buffers(i) for i in range(len(CASES))]
for i in range(len(CASES)):
    run(i, torch.cuda.current_stream(), seq[i])
torch.cuda.synchronize()
for i in range(len(CASES)):
    for kind in range(2):
        for r in range(REPS):
            assert torch.equal(par[i][kind][r], seq[i][kind][0]), (CASES[i], kind, r)
B, H, W, nh, M, s = CASES[0]
ref = oracle.swin_wattn_fwd(inputs[0][0], inputs[0][2].cpu().numpy(), M, s)
err = np.abs(par[0][0][0].float().cpu().numpy().astype(np.float64) - ref)
assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
print("threads ok", flush=True)
'''


def test_concurrent_calls_from_threads_match_sequential():
    print("[case] 4 host threads, own streams, forwards + linear, fresh process", flush=True)
    env = dict(os.environ, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    res = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    print(res.stdout[-2000:], res.stderr[-2000:], flush=True)
    assert res.returncode == 0 and "threads ok" in res.stdout
