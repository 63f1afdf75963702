"""The library's calls under HIP graph capture.

None of the calls allocates, synchronises or queues a memset: the backward
clears the table gradient with a fill kernel.  So a chain of them can be
captured once and replayed.  The test captures the attention half of a
Swin block in bf16:
- QKV projection;
- window attention;
- output projection with bias and residual;
- the attention's backward.

It then replays the graph several times, each time after new inputs were
copied into the captured buffers and some eager work ran, and compares
every replay with the same chain run eagerly.  Each step is a fixed
sequence of kernels, so every output must match bit for bit, except the
table gradient: its atomic sums vary in order, so it is compared within
fp32 rounding.  Every case prints its name before touching the GPU."""
import numpy as np
import pytest
import torch

import shifted_window_attention_swin_amd as swa
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def test_block_graph_replays_match_eager():
    B, H, W, nh, M, s = 2, 28, 28, 6, 7, 3
    C, T = nh * 32, B * H * W
    _say(f"graph capture of QKV -> attention -> projection -> backward, B={B} {H}x{W} C={C}")
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    _, w_qkv, b_qkv, _ = synth.make_linear_inputs(T, C, 3 * C, 71, False)
    _, w_p, b_p, _ = synth.make_linear_inputs(T, C, C, 72, False)
    table = torch.from_numpy(synth.attention_table(73, nh, M)).to(dev)
    pq, pp = torch.empty_like(bf(w_qkv)), torch.empty_like(bf(w_p))
    swa.check(swa.swin_linear_pack_weight(bf(w_qkv), pq, 3 * C, C), "pack qkv")
    swa.check(swa.swin_linear_pack_weight(bf(w_p), pp, C, C), "pack proj")
    bq, bp = torch.from_numpy(b_qkv).to(dev), torch.from_numpy(b_p).to(dev)

    # static buffers of the captured chain
    x = torch.empty(T, C, dtype=torch.bfloat16, device=dev)
    res = torch.empty(T, C, dtype=torch.bfloat16, device=dev)
    dout = torch.empty(B, H, W, C, dtype=torch.bfloat16, device=dev)
    qkv = torch.empty(T, 3 * C, dtype=torch.bfloat16, device=dev)
    att = torch.empty(B, H, W, C, dtype=torch.bfloat16, device=dev)
    y = torch.empty(T, C, dtype=torch.bfloat16, device=dev)
    dqkv = torch.empty(T, 3 * C, dtype=torch.bfloat16, device=dev)
    dtab = torch.empty_like(table)

    def chain():
        st = torch.cuda.current_stream()
        swa.check(swa.swin_linear_fwd(x, pq, bq, None, qkv, T, C, 3 * C, st), "qkv")
        swa.check(swa.swin_wattn_fwd(qkv, table, att, B, H, W, nh, 32, M, s, st), "fwd")
        swa.check(swa.swin_linear_fwd(att, pp, bp, res, y, T, C, C, st), "proj")
        swa.check(swa.swin_wattn_bwd(qkv, table, dout, dqkv, dtab, B, H, W, nh, 32, M, s, st), "bwd")

    def inputs(k):
        xs = synth.bf16_bits(synth.normal(synth.stream_key(80 + k, 0), T * C, 1.0)).reshape(T, C)
        rs = synth.bf16_bits(synth.normal(synth.stream_key(80 + k, 1), T * C, 1.0)).reshape(T, C)
        gs = synth.bf16_bits(synth.normal(synth.stream_key(80 + k, 2), T * C, 1.0)).reshape(B, H, W, C)
        return bf(xs), bf(rs), bf(gs)

    def load(k):
        a, b, c = inputs(k)
        x.copy_(a)
        res.copy_(b)
        dout.copy_(c)

    outs = (qkv, att, y, dqkv)
    eager = {}
    for k in range(3):  # eager reference of each input set
        load(k)
        chain()
        torch.cuda.synchronize()
        eager[k] = [t.clone() for t in outs] + [dtab.clone()]

    # capture (after a warm-up on a side stream, as torch recommends)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    torch.cuda.synchronize()

    for rep in range(2):
        for k in range(3):
            load(k)
            # eager work between the replays
            junk = torch.randn(1 << 16, device=dev).sum()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.isfinite(junk).item()
            got = [t.clone() for t in outs] + [dtab.clone()]
            for name, a, b in zip(("qkv", "attention", "projection", "dqkv"), got[:4], eager[k][:4]):
                assert torch.equal(a, b), f"replay {rep}, inputs {k}: {name} differs from eager"
            gt, et = got[4].double(), eager[k][4].double()
            assert torch.max(torch.abs(gt - et)).item() <= 1e-5 * torch.max(torch.abs(et)).item() + 1e-7
