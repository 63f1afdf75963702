"""Pins of the fp64 oracle against facts that do not come from the oracle.

Every function of the oracle is checked against at least one of: a value
worked out by hand from the definition (tests/golden), a closed form, a
library routine that computes the same thing for a special case (torch.roll,
a reshape, torch's scaled_dot_product_attention in float64), brute force on a
tiny input, or an exact invariance.  Each test names the mistake it catches.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name, dtype=np.float64):
    return np.loadtxt(os.path.join(GOLDEN, name), comments="#", dtype=dtype)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- index maps

@pytest.mark.parametrize("shape,shifts", [((2, 6, 8, 3), [(1, 2), (-3, -3), (0, 5), (-7, 4)]),
                                          ((1, 14, 14, 5), [(-3, -3), (3, 3)])])
def test_roll_matches_torch_roll(oracle_lib, shape, shifts):
    # catches a reversed shift direction or a wrong axis
    x = _rng(1).standard_normal(shape)
    for sy, sx in shifts:
        ref = torch.roll(torch.from_numpy(x), shifts=(sy, sx), dims=(1, 2)).numpy()
        assert np.array_equal(oracle.roll(x, sy, sx), ref)


@pytest.mark.parametrize("B,H,W,C,M", [(2, 14, 21, 3, 7), (1, 24, 12, 2, 12), (3, 4, 4, 1, 2)])
def test_partition_matches_reshape_and_reverses(oracle_lib, B, H, W, C, M):
    # catches transposed window or token order
    x = _rng(2).standard_normal((B, H, W, C))
    ref = (torch.from_numpy(x).view(B, H // M, M, W // M, M, C).permute(0, 1, 3, 2, 4, 5)
           .reshape(B, H // M, W // M, M * M, C).numpy())
    win = oracle.window_partition(x, M)
    assert np.array_equal(win, ref)
    assert np.array_equal(oracle.window_reverse(win, H, W, M), x)


def test_shift_then_partition_golden(oracle_lib):
    # hand-worked 4x4 example: pins the shift direction of the whole gather
    img = np.arange(16, dtype=np.float64).reshape(1, 4, 4, 1)
    win = oracle.window_partition(oracle.roll(img, -1, -1), 2)
    assert np.array_equal(win.reshape(4, 4), _golden("shift_partition_h4w4_m2_s1.txt"))


def test_shift_and_reverse_roundtrip(oracle_lib):
    x = _rng(3).standard_normal((2, 14, 14, 4))
    for s in range(7):
        back = oracle.roll(oracle.window_reverse(oracle.window_partition(oracle.roll(x, -s, -s), 7),
                                                 14, 14, 7), s, s)
        assert np.array_equal(back, x)


# --------------------------------------------------------- relative position

def test_rel_index_golden_m2(oracle_lib):
    assert np.array_equal(oracle.rel_index(2), _golden("rel_index_m2.txt", np.int32))


@pytest.mark.parametrize("M", range(1, 13))
def test_rel_index_closed_forms(oracle_lib, M):
    idx = oracle.rel_index(M)
    N, T = M * M, (2 * M - 1) ** 2
    assert idx.min() >= 0 and idx.max() <= T - 1
    # the diagonal (zero offset) sits at the centre of the table: 84 for M=7, 264 for M=12
    assert np.all(np.diag(idx) == (M - 1) * (2 * M - 1) + (M - 1))
    # opposite offsets mirror through the centre
    assert np.all(idx + idx.T == T - 1)
    # every one of the (2M-1)^2 offsets appears, and only offsets decide the index
    assert len(np.unique(idx)) == T
    ty, tx = np.divmod(np.arange(N), M)
    off = (ty[:, None] - ty[None, :]) * 100 + (tx[:, None] - tx[None, :])
    pairs = set(zip(off.ravel().tolist(), idx.ravel().tolist()))
    assert len(pairs) == T


def test_rel_index_known_values(oracle_lib):
    assert oracle.rel_index(7)[0, 0] == 84
    assert oracle.rel_index(12)[0, 0] == 264
    # query one row below the key: dy = +1, dx = 0
    idx = oracle.rel_index(7)
    assert idx[7, 0] == (1 + 6) * 13 + 6


@pytest.mark.parametrize("M", [2, 7, 12])
def test_rel_index_rank_one_difference(oracle_lib, M):
    # idx[i][j] = idx[i][0] + idx[0][j] - idx[0][0]: the index is a difference
    # of per-token codes, a structure the GPU kernel relies on
    idx = oracle.rel_index(M).astype(np.int64)
    assert np.array_equal(idx, idx[:, :1] + idx[:1, :] - idx[0, 0])


# --------------------------------------------------------------------- mask

def test_mask_golden_h4w4(oracle_lib):
    m = oracle.shift_mask(4, 4, 2, 1)
    assert np.array_equal(m.reshape(16, 4), _golden("shift_mask_h4w4_m2_s1.txt"))


@pytest.mark.parametrize("H,W,M,s", [(56, 56, 7, 3), (14, 14, 7, 3), (96, 96, 12, 6),
                                     (28, 14, 7, 2), (12, 24, 12, 5)])
def test_mask_closed_form_counts(oracle_lib, H, W, M, s):
    m = oracle.shift_mask(H, W, M, s)
    nWy, nWx, N = H // M, W // M, M * M
    assert set(np.unique(m).tolist()) <= {0.0, -100.0}
    cnt = (m == -100.0).reshape(nWy, nWx, N * N).sum(-1)
    edge = 2 * (M - s) * M * s * M
    corner = N * N - ((M - s) ** 4 + 2 * (M - s) ** 2 * s ** 2 + s ** 4)
    expect = np.zeros((nWy, nWx), dtype=np.int64)
    expect[-1, :] = edge
    expect[:, -1] = edge
    expect[-1, -1] = corner
    assert np.array_equal(cnt, expect)
    if (M, s) == (7, 3):
        assert (edge, corner) == (1176, 1776)
    if (M, s) == (12, 6):
        assert (edge, corner) == (10368, 15552)
    # the mask is symmetric and never masks a token from itself
    assert np.array_equal(m, m.transpose(0, 2, 1))
    assert np.all(np.diagonal(m, axis1=1, axis2=2) == 0.0)


def test_masked_windows_are_last_row_and_column(oracle_lib):
    """Brute force over every window size up to 8, every shift and grids of
    1-3 windows per axis: a window needs the mask exactly when the shift is
    nonzero and the window is on the last window row or column."""
    for M in range(1, 9):
        for s in range(M):
            for nWy in (1, 2, 3):
                for nWx in (1, 3):
                    m = oracle.shift_mask(nWy * M, nWx * M, M, s)
                    got = (m != 0).reshape(nWy, nWx, -1).any(-1)
                    wy, wx = np.meshgrid(np.arange(nWy), np.arange(nWx), indexing="ij")
                    expect = (s > 0) & ((wy == nWy - 1) | (wx == nWx - 1))
                    assert np.array_equal(got, expect), (M, s, nWy, nWx)


def test_mask_zero_without_shift(oracle_lib):
    assert np.all(oracle.shift_mask(56, 56, 7, 0) == 0.0)


# --------------------------------------------------------------- attention

def _torch_reference(qkv, table, M, s):
    """Library composition in float64: torch.roll, reshape partition,
    torch scaled_dot_product_attention with the additive bias+mask, reverse,
    roll back.  Index and mask come from the separately pinned oracle maps."""
    x = torch.from_numpy(np.asarray(qkv, dtype=np.float64))
    tb = torch.from_numpy(np.asarray(table, dtype=np.float64))
    return _torch_forward(x, tb, M, s).numpy()


def _torch_forward(x, tb, M, s):
    """The composition of _torch_reference on float64 tensors (differentiable)."""
    B, H, W, _, nh, d = x.shape
    N, nWy, nWx = M * M, H // M, W // M
    xr = torch.roll(x, shifts=(-s, -s), dims=(1, 2))
    win = xr.view(B, nWy, M, nWx, M, 3, nh, d).permute(0, 1, 3, 2, 4, 5, 6, 7)
    win = win.reshape(B * nWy * nWx, N, 3, nh, d)
    q, k, v = (win[:, :, i].permute(0, 2, 1, 3) for i in range(3))  # [nWin, nh, N, d]
    idx = torch.from_numpy(oracle.rel_index(M).astype(np.int64))
    bias = tb[idx]  # [N, N, nh]
    bias = bias.permute(2, 0, 1)[None]  # [1, nh, N, N]
    mask = torch.from_numpy(oracle.shift_mask(H, W, M, s)) if s > 0 else torch.zeros(1, N, N,
                                                                                     dtype=torch.float64)
    mask = mask.repeat(B, 1, 1)[:, None] if s > 0 else mask[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=bias + mask)
    o = o.permute(0, 2, 1, 3).reshape(B, nWy, nWx, M, M, nh * d).permute(0, 1, 3, 2, 4, 5)
    o = o.reshape(B, H, W, nh * d)
    return torch.roll(o, shifts=(s, s), dims=(1, 2))


@pytest.mark.parametrize("B,H,W,nh,d,M,s", [(2, 14, 14, 2, 32, 7, 3), (1, 14, 28, 3, 16, 7, 0),
                                            (1, 24, 24, 2, 32, 12, 6), (2, 8, 12, 1, 8, 4, 1)])
def test_forward_matches_torch_sdpa_float64(oracle_lib, B, H, W, nh, d, M, s):
    # catches a transposed operand, a missing scale, bias or mask, a wrong
    # softmax axis, or a wrong scatter
    q, table = synth.make_inputs(B, H, W, nh, d, M, seed=77, dtype="f32", table_std=0.5)
    out = oracle.swin_wattn_fwd(q, table, M, s)
    ref = _torch_reference(q, table, M, s)
    assert np.max(np.abs(out - ref)) < 1e-12


@pytest.mark.parametrize("L,nh,d", [(7, 2, 32), (4, 1, 8), (14, 1, 4)])
def test_window_equal_image_is_global_attention(oracle_lib, L, nh, d):
    # brute force: one window covering the whole image, no shift, zero bias
    rng = _rng(4)
    q = rng.standard_normal((1, L, L, 3, nh, d))
    table = np.zeros(((2 * L - 1) ** 2, nh), dtype=np.float32)
    out = oracle.swin_wattn_fwd(q, table, L, 0)
    tok = q.reshape(L * L, 3, nh, d)
    ref = np.empty((L * L, nh, d))
    for h in range(nh):
        Q, K, V = tok[:, 0, h], tok[:, 1, h], tok[:, 2, h]
        S = np.array([[sum(Q[i, e] * K[j, e] for e in range(d)) / math.sqrt(d)
                       for j in range(L * L)] for i in range(L * L)])
        P = np.exp(S - S.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        ref[:, h] = P @ V
    assert np.max(np.abs(out.reshape(L * L, nh, d) - ref)) < 1e-12


@pytest.mark.parametrize("s", [0, 3])
def test_softmax_rows_sum_to_one(oracle_lib, s):
    # value = 1 everywhere: each output is the sum of one softmax row
    q, table = synth.make_inputs(2, 14, 14, 2, 32, 7, seed=5, dtype="f32", table_std=1.0)
    q = q.astype(np.float64)
    q[:, :, :, 2] = 1.0
    out = oracle.swin_wattn_fwd(q, table, 7, s)
    assert np.max(np.abs(out - 1.0)) < 1e-12


def test_uniform_attention_is_window_mean(oracle_lib):
    # q = k = 0 and zero bias, no shift: every token gets the mean of v over its window
    rng = _rng(6)
    B, H, W, nh, d, M = 2, 14, 21, 2, 4, 7
    q = np.zeros((B, H, W, 3, nh, d))
    q[:, :, :, 2] = rng.standard_normal((B, H, W, nh, d))
    table = np.zeros(((2 * M - 1) ** 2, nh), dtype=np.float32)
    out = oracle.swin_wattn_fwd(q, table, M, 0).reshape(B, H, W, nh, d)
    v = q[:, :, :, 2]
    for y in range(H):
        for x in range(W):
            wy, wx = y // M, x // M
            mean = v[:, wy * M:(wy + 1) * M, wx * M:(wx + 1) * M].mean(axis=(1, 2))
            assert np.max(np.abs(out[:, y, x] - mean)) < 1e-12


def test_uniform_attention_shifted_is_region_mean(oracle_lib):
    # 4x4 image, window 2, shift 1, q = k = 0, zero bias: every token gets the
    # mean of v over the tokens of its own window that share its region; the
    # regions come from the hand-worked golden labels (masked weight e^-100)
    rng = _rng(7)
    v = rng.standard_normal((1, 4, 4, 1, 3))
    q = np.zeros((1, 4, 4, 3, 1, 3))
    q[:, :, :, 2] = v
    table = np.zeros((9, 1), dtype=np.float32)
    out = oracle.swin_wattn_fwd(q, table, 2, 1).reshape(4, 4, 3)
    labels = np.array([[0, 0, 1, 2], [0, 0, 1, 2], [3, 3, 4, 5], [6, 6, 7, 8]])  # rolled frame
    vr = np.roll(v.reshape(4, 4, 3), (-1, -1), (0, 1))  # value seen at each rolled position
    for yr in range(4):
        for xr in range(4):
            wy, wx = yr // 2, xr // 2
            members = [(a, b) for a in range(wy * 2, wy * 2 + 2) for b in range(wx * 2, wx * 2 + 2)
                       if labels[a, b] == labels[yr, xr]]
            mean = np.mean([vr[a, b] for a, b in members], axis=0)
            y, x = (yr + 1) % 4, (xr + 1) % 4
            assert np.max(np.abs(out[y, x] - mean)) < 1e-12


def test_region_labels_hand_worked(oracle_lib):
    # labels of the shifted frame, worked out by hand from the band rule
    # (per axis [0, L-M), [L-M, L-s), [L-s, L); label = 3 band_y + band_x):
    # 4x4 image, window 2, shift 1 (the frame of the region-mean test), and a
    # 6-row, 4-column image, window 2, shift 1, where the rows' bands are
    # 0 0 0 0 1 2 and the columns' 0 0 1 2
    square = np.array([[0, 0, 1, 2], [0, 0, 1, 2], [3, 3, 4, 5], [6, 6, 7, 8]])
    tall = np.array([[0, 0, 1, 2]] * 4 + [[3, 3, 4, 5], [6, 6, 7, 8]])
    assert np.array_equal(oracle.region_labels(4, 4, 2, 1), square)
    assert np.array_equal(oracle.region_labels(6, 4, 2, 1), tall)
    # no shift: one region
    assert not oracle.region_labels(6, 4, 2, 0).any()


def test_one_hot_bias_sign(oracle_lib):
    # bias +50 only for offset (dy, dx) = (+1, 0) (query one row below the key):
    # every query not in its window's first row copies the value one row above
    rng = _rng(8)
    B, H, W, nh, d, M = 1, 14, 14, 2, 4, 7
    q = np.zeros((B, H, W, 3, nh, d))
    q[:, :, :, 2] = rng.standard_normal((B, H, W, nh, d))
    table = np.zeros(((2 * M - 1) ** 2, nh), dtype=np.float32)
    table[(1 + M - 1) * (2 * M - 1) + (M - 1)] = 50.0
    out = oracle.swin_wattn_fwd(q, table, M, 0).reshape(B, H, W, nh, d)
    v = q[:, :, :, 2]
    for y in range(H):
        for x in range(W):
            if y % M == 0:
                continue
            assert np.max(np.abs(out[:, y, x] - v[:, y - 1, x])) < 1e-12


def test_linearity_in_value(oracle_lib):
    q, table = synth.make_inputs(2, 14, 14, 2, 32, 7, seed=9, dtype="f32")
    q2 = q.astype(np.float64).copy()
    q2[:, :, :, 2] *= 2.0
    assert np.array_equal(oracle.swin_wattn_fwd(q2, table, 7, 3), 2.0 * oracle.swin_wattn_fwd(q, table, 7, 3))


def test_table_offset_invariance(oracle_lib):
    q, table = synth.make_inputs(1, 14, 14, 2, 32, 7, seed=10, dtype="f32")
    # table on a 2^-16 grid so that adding 0.5 is exact in float32
    table = (np.round(table.astype(np.float64) * 2 ** 16) / 2 ** 16).astype(np.float32)
    a = oracle.swin_wattn_fwd(q, table, 7, 3)
    b = oracle.swin_wattn_fwd(q, table + np.float32(0.5), 7, 3)
    assert np.max(np.abs(a - b)) < 1e-12


@pytest.mark.parametrize("M,npad", [(7, 64), (7, 56), (12, 160), (5, 32)])
def test_padding_is_exact(oracle_lib, M, npad):
    # padded keys score -inf, so their weights are exactly zero
    q, table = synth.make_inputs(2, 2 * M, 3 * M, 2, 16, M, seed=11, dtype="bf16")
    a = oracle.swin_wattn_fwd(q, table, M, M // 2)
    b = oracle.swin_wattn_fwd(q, table, M, M // 2, npad=npad)
    assert np.array_equal(a, b)


def test_unshifted_roll_equivariance(oracle_lib):
    q, table = synth.make_inputs(1, 21, 14, 2, 8, 7, seed=12, dtype="f32")
    a = oracle.swin_wattn_fwd(q, table, 7, 0)
    qr = np.roll(q, (7, 7), (1, 2))
    b = oracle.swin_wattn_fwd(qr, table, 7, 0)
    assert np.array_equal(np.roll(a, (7, 7), (1, 2)), b)


def test_bf16_patterns_read_exactly(oracle_lib):
    q, table = synth.make_inputs(1, 14, 14, 2, 32, 7, seed=13, dtype="bf16")
    a = oracle.swin_wattn_fwd(q, table, 7, 3)
    b = oracle.swin_wattn_fwd(synth.bf16_to_f32(q).astype(np.float64), table, 7, 3)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("B,H,W,nh,M,s", [(2, 14, 14, 2, 7, 3), (1, 24, 36, 3, 12, 6), (3, 14, 14, 1, 7, 0)])
def test_selected_windows_equal_whole_forward(oracle_lib, B, H, W, nh, M, s):
    q, table = synth.make_inputs(B, H, W, nh, 32, M, seed=14, dtype="bf16")
    full = oracle.swin_wattn_fwd(q, table, M, s).reshape(B * H * W, -1)
    nW = (H // M) * (W // M)
    sel = np.arange(B * nW)[::-1].copy()
    out, pos = oracle.swin_wattn_windows(q, table, M, s, sel)
    assert np.array_equal(np.sort(pos.ravel()), np.arange(B * H * W))
    assert np.array_equal(out.reshape(-1, out.shape[-1]), full[pos.ravel()])


def test_thread_count_does_not_change_result(oracle_lib):
    q, table = synth.make_inputs(2, 14, 14, 2, 32, 7, seed=15, dtype="bf16")
    a = oracle.swin_wattn_fwd(q, table, 7, 3, nthreads=1)
    b = oracle.swin_wattn_fwd(q, table, 7, 3, nthreads=3)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- linear layer

def test_linear_golden(oracle_lib):
    x = np.array([[1, 2, 3], [-1, 0, 2]], dtype=np.float64)
    w = np.array([[1, 0, -1], [2, 1, 0]], dtype=np.float64)
    b = np.array([0.5, -1], dtype=np.float32)
    r = np.array([[10, 20], [30, 40]], dtype=np.float64)
    assert np.array_equal(oracle.linear(x, w, b, r), _golden("linear_t2_k3_n2.txt"))


@pytest.mark.parametrize("T,K,N,with_bias,with_res", [(1, 1, 1, True, False), (37, 96, 288, True, False),
                                                       (64, 192, 576, True, False),
                                                       (50, 192, 192, True, True), (9, 32, 64, False, True),
                                                       (0, 32, 96, True, True)])
def test_linear_matches_numpy_float64(oracle_lib, T, K, N, with_bias, with_res):
    """Special case reducing to a library routine: numpy's float64 matmul."""
    rng = _rng(T * 7 + K + N)
    x, w = rng.standard_normal((T, K)), rng.standard_normal((N, K)) * 0.05
    b = rng.standard_normal(N).astype(np.float32) if with_bias else None
    r = rng.standard_normal((T, N)) if with_res else None
    ref = x @ w.T
    if with_bias:
        ref = ref + b.astype(np.float64)
    if with_res:
        ref = ref + r
    got = oracle.linear(x, w, b, r)
    assert got.shape == (T, N)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_linear_identity_and_one_hot(oracle_lib):
    """Closed forms: w = I gives x + bias exactly; a one-hot row j -> c copies
    input channel c to output j (a transposed operand would fail this)."""
    rng = _rng(5)
    x = rng.standard_normal((11, 8))
    b = rng.standard_normal(8).astype(np.float32)
    assert np.array_equal(oracle.linear(x, np.eye(8), b), x + b.astype(np.float64))
    w = np.zeros((3, 8))
    w[0, 5] = w[1, 0] = w[2, 7] = 1.0
    assert np.array_equal(oracle.linear(x, w), x[:, [5, 0, 7]])


def test_linear_bf16_read_exactly(oracle_lib):
    rng = _rng(6)
    x = synth.bf16_bits(rng.standard_normal((13, 32)).astype(np.float32))
    w = synth.bf16_bits((rng.standard_normal((64, 32)) * 0.02).astype(np.float32))
    r = synth.bf16_bits(rng.standard_normal((13, 64)).astype(np.float32))
    xf, wf, rf = (synth.bf16_to_f32(a).astype(np.float64) for a in (x, w, r))
    assert np.array_equal(oracle.linear(x, w, None, r), oracle.linear(xf, wf, None, rf))


def test_linear_thread_count_does_not_change_result(oracle_lib):
    rng = _rng(8)
    x, w = rng.standard_normal((101, 64)), rng.standard_normal((96, 64))
    assert np.array_equal(oracle.linear(x, w, nthreads=1), oracle.linear(x, w, nthreads=7))


def test_qkv_columns_are_the_attention_layout(oracle_lib):
    """Reading: the QKV projection's N = 3C outputs are ordered [3][heads][d],
    so reshaping a token row to (3, heads, d) gives q, k, v per head; output
    row (i, h, e) of the weight produces component i of head h, channel e."""
    rng = _rng(9)
    nh, d, C = 3, 32, 96
    x = rng.standard_normal((2, 4, 4, C))
    w = rng.standard_normal((3 * C, C)) * 0.05
    b = rng.standard_normal(3 * C).astype(np.float32)
    qkv = oracle.linear(x, w, b).reshape(2, 4, 4, 3, nh, d)
    for i in range(3):
        for h in range(nh):
            rows = slice((i * nh + h) * d, (i * nh + h + 1) * d)
            ref = x @ w[rows].T + b[rows].astype(np.float64)
            assert np.allclose(qkv[:, :, :, i, h, :], ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- layer norm

def test_layernorm_golden(oracle_lib):
    x = np.array([1.0, 2.0, 3.0, 4.0])
    y1 = oracle.layernorm(x[None], np.ones(4, np.float32), np.zeros(4, np.float32), eps=0.0)
    y2 = oracle.layernorm(x[None], np.array([2, 1, 1, 1], np.float32),
                          np.array([0, 0, 0, 1], np.float32), eps=0.0)
    g = _golden("layernorm_c4.txt")
    assert np.allclose(y1[0], g[0], rtol=0, atol=1e-14)
    assert np.allclose(y2[0], g[1], rtol=0, atol=1e-14)


@pytest.mark.parametrize("T,C,eps", [(1, 1, 1e-5), (9, 96, 1e-5), (33, 192, 1e-6), (5, 384, 1e-3)])
def test_layernorm_matches_torch_float64(oracle_lib, T, C, eps):
    """Special case reducing to a library routine: torch's layer_norm in float64."""
    rng = _rng(T + C)
    x = rng.standard_normal((T, C)) * 3 + 1.5
    g, b = rng.standard_normal(C).astype(np.float32), rng.standard_normal(C).astype(np.float32)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (C,), torch.from_numpy(g.astype(np.float64)),
                                         torch.from_numpy(b.astype(np.float64)), eps).numpy()
    assert np.allclose(oracle.layernorm(x, g, b, eps), ref, rtol=1e-12, atol=1e-12)


def test_layernorm_closed_forms(oracle_lib):
    rng = _rng(12)
    C = 64
    ones, zeros = np.ones(C, np.float32), np.zeros(C, np.float32)
    b = rng.standard_normal(C).astype(np.float32)
    # a constant row has zero variance: the output is beta
    assert np.array_equal(oracle.layernorm(np.full((3, C), 7.25), ones, b, eps=1e-5),
                          np.broadcast_to(b.astype(np.float64), (3, C)))
    # unit scale, zero shift: each row has mean 0 and variance var / (var + eps)
    x = rng.standard_normal((6, C)) * 2 + 5
    y = oracle.layernorm(x, ones, zeros, eps=0.5)
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-13)
    assert np.allclose(y.var(axis=1), var / (var + 0.5), rtol=1e-12)
    # without eps the result is invariant under x -> a x + c, a > 0
    assert np.allclose(oracle.layernorm(3 * x - 11, ones, b, eps=0.0),
                       oracle.layernorm(x, ones, b, eps=0.0), rtol=1e-12, atol=1e-12)


def test_layernorm_bf16_read_exactly(oracle_lib):
    rng = _rng(13)
    xb = synth.bf16_bits(rng.standard_normal((5, 96)).astype(np.float32))
    g, b = rng.standard_normal(96).astype(np.float32), rng.standard_normal(96).astype(np.float32)
    assert np.array_equal(oracle.layernorm(xb, g, b), oracle.layernorm(synth.bf16_to_f32(xb).astype(np.float64), g, b))



# ---------------------------------------------------------------- backward

@pytest.mark.parametrize("B,H,W,nh,d,M,s", [(2, 14, 14, 2, 32, 7, 3), (1, 14, 28, 3, 16, 7, 0),
                                            (1, 24, 24, 2, 32, 12, 6), (2, 8, 12, 1, 8, 4, 1)])
def test_backward_matches_torch_autograd_float64(oracle_lib, B, H, W, nh, d, M, s):
    """Special case reducing to a library routine: torch autograd of the
    float64 composition, for the gradients of qkv and of the bias table."""
    q, table = synth.make_inputs(B, H, W, nh, d, M, seed=78, dtype="f32", table_std=0.5)
    g = _rng(79).standard_normal((B, H, W, nh * d))
    dq, dt = oracle.swin_wattn_bwd(q, table, g, M, s)
    x = torch.from_numpy(np.asarray(q, dtype=np.float64)).requires_grad_(True)
    tb = torch.from_numpy(np.asarray(table, dtype=np.float64)).requires_grad_(True)
    (_torch_forward(x, tb, M, s) * torch.from_numpy(g)).sum().backward()
    assert np.max(np.abs(dq - x.grad.numpy())) < 1e-11
    assert np.max(np.abs(dt - tb.grad.numpy())) < 1e-10


def test_backward_finite_differences(oracle_lib):
    """Brute force: central differences of L = sum(out * g) on a tiny case
    (shifted, masked windows), for sampled qkv entries and every table entry."""
    B, H, W, nh, d, M, s = 1, 4, 4, 2, 3, 2, 1
    rng = _rng(80)
    q = rng.standard_normal((B, H, W, 3, nh, d))
    table = (rng.standard_normal(((2 * M - 1) ** 2, nh)) * 0.5).astype(np.float32)
    g = rng.standard_normal((B, H, W, nh * d))
    dq, dt = oracle.swin_wattn_bwd(q, table, g, M, s)
    L = lambda qq, tt: float((oracle.swin_wattn_fwd(qq, tt, M, s) * g).sum())
    h = 1e-6
    flat = q.reshape(-1)
    for i in rng.choice(flat.size, 40, replace=False):
        qp, qm = flat.copy(), flat.copy()
        qp[i] += h
        qm[i] -= h
        fd = (L(qp.reshape(q.shape), table) - L(qm.reshape(q.shape), table)) / (2 * h)
        assert abs(fd - dq.reshape(-1)[i]) < 1e-6 * max(1.0, abs(fd))
    # the table is fp32 in the oracle: a step of 2^-12 on entries of size < 2
    # is exact in fp32, and the difference quotient is then accurate to ~1e-6
    hs = 2.0 ** -12
    for i in range(table.size):
        tp, tm = table.copy().reshape(-1), table.copy().reshape(-1)
        tp[i] += hs
        tm[i] -= hs
        fd = (L(q, tp.reshape(table.shape)) - L(q, tm.reshape(table.shape))) / (2 * hs)
        assert abs(fd - dt.reshape(-1)[i]) < 1e-5 * max(1.0, abs(fd))


def test_backward_invariants(oracle_lib):
    """Every row of dS sums to zero (the softmax Jacobian annihilates
    constants), so the table gradient of each head sums to zero; the
    gradients are linear in dout; with v = 0, dP = dO V^T = 0, so dS = 0:
    dQ, dK and the table gradient vanish while dV = P^T dO does not."""
    B, H, W, nh, d, M, s = 2, 14, 14, 3, 8, 7, 3
    q, table = synth.make_inputs(B, H, W, nh, d, M, seed=81, dtype="f32", table_std=0.3)
    g = _rng(82).standard_normal((B, H, W, nh * d))
    dq, dt = oracle.swin_wattn_bwd(q, table, g, M, s)
    assert np.all(np.abs(dt.sum(axis=0)) < 1e-10)
    dq2, dt2 = oracle.swin_wattn_bwd(q, table, 2 * g, M, s)
    assert np.allclose(dq2, 2 * dq, rtol=1e-12, atol=1e-13) and np.allclose(dt2, 2 * dt, rtol=1e-12, atol=1e-13)
    q0 = np.array(q, dtype=np.float64)
    q0[:, :, :, 2] = 0.0
    dq0, dt0 = oracle.swin_wattn_bwd(q0, table, g, M, s)
    assert np.all(dq0[:, :, :, :2] == 0.0) and np.all(dt0 == 0.0)
    assert np.any(dq0[:, :, :, 2] != 0.0)


# ------------------------------------------------------------------- INT8

def test_dequant_qkv_i8_golden(oracle_lib):
    # hand-worked: catches a scale applied to the wrong part
    codes = np.array([[-127, 3], [0, 127], [-1, 64]], dtype=np.int8).reshape(1, 3, 1, 2)
    got = oracle.dequant_qkv_i8(codes, [0.5, 0.25, 2.0])
    assert np.array_equal(got.reshape(3, 2), _golden("dequant_qkv_i8_c2.txt"))


@pytest.mark.parametrize("B,H,W,nh,M,s", [(2, 14, 14, 2, 7, 3), (1, 24, 24, 3, 12, 6), (1, 8, 12, 1, 4, 0)])
def test_forward_i8_matches_torch_sdpa_float64(oracle_lib, B, H, W, nh, M, s):
    # the codes dequantized by torch broadcasting, then the library
    # composition: catches a scale taken from the wrong part or a code read
    # as unsigned
    codes, scales, table = synth.make_i8_inputs(B, H, W, nh, 32, M, seed=91 + M,
                                                scales=(0.05, 0.02, 0.07))
    codes[0, 0, 0, :, 0, :3] = np.array([-128, 127, -1], dtype=np.int8)  # the extreme codes
    sc = torch.tensor(scales.astype(np.float64)).view(3, 1, 1)
    x = torch.from_numpy(codes.astype(np.int64)).double() * sc
    ref = _torch_reference(x.numpy(), table, M, s)
    got = oracle.swin_wattn_fwd_i8(codes, scales, table, M, s)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_forward_i8_scale_invariances(oracle_lib):
    # exact invariances of the definition: the scores see only the product of
    # the query and key scales, and the output is linear in the value scale.
    # Catches the value scale applied to the query or key (then the output
    # would not scale linearly) and a query or key scale that is dropped.
    codes, _, table = synth.make_i8_inputs(1, 14, 14, 2, 32, 7, seed=95)
    base = oracle.swin_wattn_fwd_i8(codes, [0.04, 0.03, 0.02], table, 7, 3)
    swapped = oracle.swin_wattn_fwd_i8(codes, [0.16, 0.0075, 0.02], table, 7, 3)
    assert np.max(np.abs(swapped - base)) < 1e-12
    tripled = oracle.swin_wattn_fwd_i8(codes, [0.04, 0.03, 0.06], table, 7, 3)
    assert np.max(np.abs(tripled - 3 * base)) < 1e-12
    sharper = oracle.swin_wattn_fwd_i8(codes, [0.08, 0.03, 0.02], table, 7, 3)
    assert np.max(np.abs(sharper - base)) > 1e-3


def test_linear_i8_golden(oracle_lib):
    # hand-worked: ties to even and saturation at +-127 (never -128)
    x = np.array([[3, -2], [5, 7]], dtype=np.int8)
    w = np.array([[10, 20], [-7, 1], [1, 0], [-127, 127]], dtype=np.int8)
    acc, y, yq = oracle.linear_i8(x, 0.5, w, [0.25, 2, 1, 1], bias=[0.5, -1, 0, 0],
                                  so=[1, 4, 1, 0.25])
    g = _golden("linear_i8_t2_k2_n4.txt")
    assert np.array_equal(acc, np.array([[-10, -23, 3, -635], [190, -28, 5, 254]]))
    assert np.array_equal(y, g[:2]) and np.array_equal(yq.astype(np.float64), g[2:])


@pytest.mark.parametrize("T,K,N,with_res", [(37, 96, 288, False), (64, 192, 576, True), (5, 1536, 64, False)])
def test_linear_i8_matches_numpy(oracle_lib, T, K, N, with_res):
    # exact integer sums against numpy's int64 product; the dequantized value
    # against numpy float64; catches a transposed weight, a per-channel scale
    # taken by input channel, or a dropped bias or residual
    x = synth.int8_codes(synth.stream_key(7, 0), T * K).reshape(T, K)
    w = synth.int8_codes(synth.stream_key(7, 1), N * K).reshape(N, K)
    sw = np.abs(synth.normal(synth.stream_key(7, 2), N, 1e-3)) + np.float32(1e-4)
    b = synth.normal(synth.stream_key(7, 3), N, 0.1)
    r = synth.normal(synth.stream_key(7, 4), T * N, 1.0).reshape(T, N) if with_res else None
    acc, y, _ = oracle.linear_i8(x, 0.02, w, sw, bias=b, residual=r)
    ref_acc = x.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(acc, ref_acc)
    ref = ref_acc.astype(np.float64) * 0.019999999552965164 * sw.astype(np.float64) + b
    if with_res:
        ref = ref + r
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_linear_i8_codes_round_the_value(oracle_lib):
    # the fp32 decision may differ from rounding the fp64 value only at a
    # near-tie: every code is within 1/2 (plus fp32 rounding) of y / so and
    # equals the rounded fp64 value away from ties; codes saturate at +-127
    T, K, N = 256, 192, 96
    x = synth.int8_codes(synth.stream_key(8, 0), T * K).reshape(T, K)
    w = synth.int8_codes(synth.stream_key(8, 1), N * K).reshape(N, K)
    sw = np.abs(synth.normal(synth.stream_key(8, 2), N, 1e-3)) + np.float32(1e-4)
    b = synth.normal(synth.stream_key(8, 3), N, 0.5)
    so = np.abs(synth.normal(synth.stream_key(8, 4), N, 0.02)) + np.float32(0.005)
    so[:8] = 1e-4  # columns that saturate
    acc, y, yq = oracle.linear_i8(x, 0.015, w, sw, bias=b, so=so)
    v = y / so.astype(np.float64)
    exact = np.clip(np.rint(v), -127, 127)
    got = yq.astype(np.float64)
    assert np.all(np.abs(got - exact) <= 1)
    inside = np.abs(v) < 126
    assert np.all(np.abs(got[inside] - v[inside]) <= 0.5 + 1e-5 * np.abs(v[inside]) + 1e-6)
    far = np.abs(np.abs(v - np.floor(v)) - 0.5) > 1e-3
    assert np.array_equal(got[far], exact[far])
    sat = np.abs(v) >= 127.5
    assert sat[:, :8].mean() > 0.9 and np.array_equal(got[sat], 127 * np.sign(v[sat]))
    assert got.min() >= -127
