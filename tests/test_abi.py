"""The C ABI without a GPU: the library loads, exports every function that
include/swinattn.h declares, and rejects bad arguments with the documented
status before any device call."""
import os
import re
import subprocess

import pytest

import shifted_window_attention_swin_amd as swa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swinattn.h")

# aligned, non-null placeholder addresses: argument checks reject the call
# before anything dereferences them
A16, A32, A48 = 1 << 20, 2 << 20, 3 << 20


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*|void)\s+(swin_\w+)\s*\(", src, re.M)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(swa.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", swa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(swin_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(swa.library(), name)


def test_status_strings():
    for code in (swa.SWIN_OK, swa.SWIN_ERR_INVALID_ARG, swa.SWIN_ERR_UNSUPPORTED,
                 swa.SWIN_ERR_NOT_PREPARED, swa.SWIN_ERR_HIP):
        assert swa.swin_wattn_status_string(code).startswith("SWIN_")
    assert swa.swin_wattn_status_string(12345) == "unknown status"


GOOD = dict(B=2, H=14, W=14, heads=2, head_dim=32, window=7, shift=3)


def _fwd_i8(qkv, table, out, *rest):
    """swin_wattn_fwd_i8 with valid scales, in the argument order of swin_wattn_fwd."""
    return swa.swin_wattn_fwd_i8(qkv, 0.03, 0.03, 0.03, 0.0, table, out, *rest)


FWDS = [swa.swin_wattn_fwd, swa.swin_wattn_fwd_f32, _fwd_i8]


def _fwd(fn=None, qkv=A16, table=A32, out=A48, **kw):
    a = dict(GOOD)
    a.update(kw)
    fn = fn or swa.swin_wattn_fwd
    return fn(qkv, table, out, a["B"], a["H"], a["W"], a["heads"], a["head_dim"], a["window"],
              a["shift"], 0)


@pytest.mark.parametrize("fn", FWDS)
def test_fwd_rejects_invalid_arguments(fn):
    E = swa.SWIN_ERR_INVALID_ARG
    assert _fwd(fn, qkv=0) == E
    assert _fwd(fn, table=0) == E
    assert _fwd(fn, out=0) == E
    assert _fwd(fn, qkv=A16 + 8) == E          # not 16-byte aligned
    assert _fwd(fn, out=A48 + 4) == E
    assert _fwd(fn, table=A32 + 2) == E        # not 4-byte aligned
    assert _fwd(fn, B=-1) == E
    assert _fwd(fn, H=0) == E
    assert _fwd(fn, W=-7) == E
    assert _fwd(fn, heads=0) == E
    assert _fwd(fn, H=15) == E                 # H % window != 0
    assert _fwd(fn, W=20) == E
    assert _fwd(fn, shift=7) == E              # shift >= window
    assert _fwd(fn, shift=-1) == E
    assert _fwd(fn, window=0) == E
    assert _fwd(fn, out=A16) == E              # out overlaps qkv


@pytest.mark.parametrize("fn", FWDS)
def test_fwd_reports_unsupported_configurations(fn):
    U = swa.SWIN_ERR_UNSUPPORTED
    assert _fwd(fn, head_dim=64) == U
    assert _fwd(fn, head_dim=16) == U
    assert _fwd(fn, window=14, shift=0) == U


def test_fp32_fwd_reports_bias_tables_beyond_lds():
    # the fp32 kernel stages every head's table: 78 heads at window 12 are
    # 165,048 bytes, beyond the 160 KiB of LDS a workgroup may use (the bf16
    # forward takes any number of heads; a call with valid arguments cannot
    # be made here, since these placeholder pointers must never reach a
    # kernel)
    U = swa.SWIN_ERR_UNSUPPORTED
    assert _fwd(swa.swin_wattn_fwd_f32, window=12, H=24, W=24, shift=0, heads=78) == U


@pytest.mark.parametrize("fn", FWDS)
def test_empty_batch_is_a_no_op(fn):
    assert _fwd(fn, B=0) == swa.SWIN_OK


def test_fwd_i8_rejects_scales_out_of_range():
    E = swa.SWIN_ERR_INVALID_ARG

    def call(sq, sk, sv, so=0.0):
        return swa.swin_wattn_fwd_i8(A16, sq, sk, sv, so, A32, A48, 2, 14, 14, 2, 32, 7, 3, 0)

    nan, inf = float("nan"), float("inf")
    for bad in [(0.0, 0.03, 0.03), (0.03, -0.03, 0.03), (0.03, 0.03, 0.0), (nan, 0.03, 0.03),
                (0.03, nan, 0.03), (0.03, 0.03, nan), (inf, 0.03, 0.03), (0.03, 0.03, inf),
                (1e-20, 1e-20, 1.0),     # score scale below 2^-100
                (1e20, 1e20, 1.0),       # score scale above 2^100
                (1.0, 1.0, 2.0 ** 101),
                (0.03, 0.03, 0.03, -1.0),      # negative output scale
                (0.03, 0.03, 0.03, nan),
                (0.03, 0.03, 1e20, 1e-20)]:    # scale_v / out_scale above 2^100
        assert call(*bad) == E, bad
    # near the range's ends: accepted (B = 0: nothing is queued)
    lo, hi = 2.0 ** -48, 2.0 ** 50
    assert swa.swin_wattn_fwd_i8(A16, lo, lo, 2.0 ** 100, 0.0, A32, A48, 0, 14, 14, 2, 32, 7, 3, 0) == 0
    assert swa.swin_wattn_fwd_i8(A16, hi, hi, 1.0, 0.0, A32, A48, 0, 14, 14, 2, 32, 7, 3, 0) == 0
    assert swa.swin_wattn_fwd_i8(A16, 0.03, 0.03, 0.03, 0.01, A32, A48, 0, 14, 14, 2, 32, 7, 3, 0) == 0


def test_precompute_and_copies_reject_invalid_shapes():
    E = swa.SWIN_ERR_INVALID_ARG
    assert swa.swin_wattn_precompute(14, 14, 7, 7) == E
    assert swa.swin_wattn_precompute(14, 15, 7, 3) == E
    assert swa.swin_wattn_precompute(0, 14, 7, 3) == E
    assert swa.swin_wattn_precompute(26, 26, 13, 0) == E
    assert swa.swin_wattn_precompute(14, 14, 0, 0) == E
    for fn in (swa.swin_wattn_copy_index, swa.swin_wattn_copy_mask, swa.swin_wattn_copy_region):
        assert fn(14, 14, 7, 3, 0) == E
        assert fn(14, 14, 7, 9, A16) == E


def test_linear_rejects_invalid_arguments():
    E, U = swa.SWIN_ERR_INVALID_ARG, swa.SWIN_ERR_UNSUPPORTED
    a, b, c = 1 << 20, 2 << 20, 3 << 20      # aligned, distinct, never dereferenced
    assert swa.swin_linear_fwd(0, b, None, None, c, 64, 192, 576) == E          # null x
    assert swa.swin_linear_fwd(a, 0, None, None, c, 64, 192, 576) == E          # null weight
    assert swa.swin_linear_fwd(a, b, None, None, 0, 64, 192, 576) == E          # null y
    assert swa.swin_linear_fwd(a + 8, b, None, None, c, 64, 192, 576) == E      # misaligned x
    assert swa.swin_linear_fwd(a, b, a + 4, None, c, 64, 192, 576) == E         # misaligned bias
    assert swa.swin_linear_fwd(a, b, None, c + 8, c, 64, 192, 576) == E         # misaligned residual
    assert swa.swin_linear_fwd(a, b, None, None, c, -1, 192, 576) == E          # negative T
    assert swa.swin_linear_fwd(a, b, None, None, c, 64, 100, 576) == E          # K % 32
    assert swa.swin_linear_fwd(a, b, None, None, c, 64, 192, 500) == E          # N % 32
    assert swa.swin_linear_fwd(a, b, None, None, c, 64, 0, 576) == E
    assert swa.swin_linear_fwd(a, b, None, None, c, 64, 416, 576) == U          # K > 384
    assert swa.swin_linear_fwd(a, b, None, None, a, 64, 192, 576) == E          # y overlaps x
    assert swa.swin_linear_fwd(a, b, None, c + 64, c, 64, 192, 576) == E        # residual overlaps y
    assert swa.swin_linear_pack_weight(0, b, 576, 192) == E
    assert swa.swin_linear_pack_weight(a, b, 576, 100) == E
    assert swa.swin_linear_pack_weight(a, b, 500, 192) == E
    assert swa.swin_linear_pack_weight(a, a, 576, 192) == E                     # packed overlaps W
    assert swa.swin_linear_pack_weight(a, b, 576, 416) == U


def test_linear_i8_rejects_invalid_arguments():
    E, U = swa.SWIN_ERR_INVALID_ARG, swa.SWIN_ERR_UNSUPPORTED
    a, b, c, ws, os_ = 1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20  # aligned, never dereferenced

    def call(x=a, sx=0.03, wp=b, sw=ws, bias=None, res=None, so=None, y=c, T=64, K=192, N=576):
        return swa.swin_linear_i8_fwd(x, sx, wp, sw, bias, res, so, y, T, K, N)

    assert call(x=0) == E
    assert call(wp=0) == E
    assert call(sw=0) == E                  # the weight scales are required
    assert call(y=0) == E
    assert call(x=a + 8) == E               # misaligned
    assert call(sw=ws + 4) == E
    assert call(so=os_ + 8) == E
    assert call(bias=a + 4) == E
    assert call(sx=0.0) == E                # x scale must be finite and > 0
    assert call(sx=-1.0) == E
    assert call(sx=float("nan")) == E
    assert call(sx=float("inf")) == E
    assert call(res=c, so=os_) == E         # no residual with int8 output
    assert call(T=-1) == E
    assert call(K=100) == E                 # K % 32
    assert call(N=500) == E                 # N % 32
    assert call(K=800) == U                 # K > 768
    assert call(y=a) == E                   # y overlaps x
    assert call(y=ws - 64, T=1, N=64) == E  # y overlaps the weight scales
    assert call(T=0) == swa.SWIN_OK
    assert call(T=0, so=os_, K=96) == swa.SWIN_OK
    assert swa.swin_linear_i8_pack_weight(0, b, 576, 192) == E
    assert swa.swin_linear_i8_pack_weight(a, b, 576, 100) == E
    assert swa.swin_linear_i8_pack_weight(a, b, 500, 192) == E
    assert swa.swin_linear_i8_pack_weight(a, a, 576, 192) == E   # packed overlaps W
    assert swa.swin_linear_i8_pack_weight(a, b, 576, 800) == U


def test_linear_empty_is_a_no_op():
    assert swa.swin_linear_fwd(1 << 20, 2 << 20, None, None, 3 << 20, 0, 192, 576) == swa.SWIN_OK
    # in-place residual (residual == y) is accepted
    assert swa.swin_linear_fwd(1 << 20, 2 << 20, None, 3 << 20, 3 << 20, 0, 192, 192) == swa.SWIN_OK


def test_ln_linear_rejects_invalid_arguments():
    E, U = swa.SWIN_ERR_INVALID_ARG, swa.SWIN_ERR_UNSUPPORTED
    a, b, c, k, g, be = 1 << 20, 2 << 20, 3 << 20, 6 << 20, 4 << 20, 5 << 20
    assert swa.swin_ln_linear_fwd(a, b, 0, 1e-5, c, 64, 192, 576) == E          # null consts
    assert swa.swin_ln_linear_fwd(a, b, k + 4, 1e-5, c, 64, 192, 576) == E      # misaligned consts
    assert swa.swin_ln_linear_fwd(a, b, k, -1.0, c, 64, 192, 576) == E          # negative eps
    assert swa.swin_ln_linear_fwd(a, b, k, float("nan"), c, 64, 192, 576) == E
    assert swa.swin_ln_linear_fwd(a, b, k, 1e-5, c, 64, 100, 576) == E          # K % 32
    assert swa.swin_ln_linear_fwd(a, b, k, 1e-5, c, 64, 416, 576) == U          # K > 384
    assert swa.swin_ln_linear_fwd(a, b, k, 1e-5, k, 64, 192, 576) == E          # y overlaps consts
    assert swa.swin_ln_linear_fwd(a, b, k, 1e-5, c, 0, 192, 576) == swa.SWIN_OK
    assert swa.swin_ln_linear_pack_weight(a, 0, be, None, b, k, 576, 192) == E  # null gamma
    assert swa.swin_ln_linear_pack_weight(a, g, 0, None, b, k, 576, 192) == E   # null beta
    assert swa.swin_ln_linear_pack_weight(a, g, be, None, b, 0, 576, 192) == E  # null consts
    assert swa.swin_ln_linear_pack_weight(a, g, be, None, b, k + 8, 576, 192) == E
    assert swa.swin_ln_linear_pack_weight(a, g, be, None, b, b, 576, 192) == E  # consts overlap packed
    assert swa.swin_ln_linear_pack_weight(a, g, be, None, b, k, 576, 100) == E
    assert swa.swin_ln_linear_pack_weight(a, g, be, None, b, k, 576, 416) == U


def _bwd(**kw):
    a = dict(qkv=A16, table=A32, dout=A48, dqkv=4 << 20, dtable=5 << 20, B=2, H=14, W=14,
             heads=3, head_dim=32, window=7, shift=3)
    a.update(kw)
    return swa.swin_wattn_bwd(a["qkv"], a["table"], a["dout"], a["dqkv"], a["dtable"], a["B"],
                              a["H"], a["W"], a["heads"], a["head_dim"], a["window"], a["shift"], 0)


def test_bwd_rejects_invalid_arguments():
    E = swa.SWIN_ERR_INVALID_ARG
    for k in ("qkv", "table", "dout", "dqkv", "dtable"):
        assert _bwd(**{k: 0}) == E, k
    assert _bwd(qkv=A16 + 8) == E              # not 16-byte aligned
    assert _bwd(dout=A48 + 8) == E
    assert _bwd(dqkv=(4 << 20) + 4) == E
    assert _bwd(dtable=(5 << 20) + 2) == E     # not 4-byte aligned
    assert _bwd(B=-1) == E
    assert _bwd(H=15) == E
    assert _bwd(shift=7) == E
    assert _bwd(window=0) == E
    assert _bwd(dqkv=A16) == E                 # dqkv overlaps qkv
    assert _bwd(dtable=A48 + 64) == E          # dtable overlaps dout
    assert _bwd(dtable=A32) == E               # dtable overlaps the table


def test_bwd_reports_unsupported_configurations():
    U = swa.SWIN_ERR_UNSUPPORTED
    assert _bwd(head_dim=64) == U
    assert _bwd(window=13, H=26, W=26, shift=6) == U        # windows beyond 12


def test_ln_qkv_wattn_rejects_invalid_arguments():
    E, U = swa.SWIN_ERR_INVALID_ARG, swa.SWIN_ERR_UNSUPPORTED
    a, b, c, d, o = 1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20  # aligned, never dereferenced

    def call(x=a, wp=b, cs=c, eps=1e-5, tab=d, out=o, B=2, H=14, W=14, heads=6, hd=32, M=7, s=3):
        return swa.swin_ln_qkv_wattn_fwd(x, wp, cs, eps, tab, out, B, H, W, heads, hd, M, s)

    assert call(x=0) == E
    assert call(wp=0) == E
    assert call(cs=0) == E
    assert call(tab=0) == E
    assert call(out=0) == E
    assert call(x=a + 8) == E          # misaligned
    assert call(cs=c + 4) == E
    assert call(tab=d + 2) == E
    assert call(eps=-1.0) == E
    assert call(B=-1) == E
    assert call(H=15) == E             # H % window
    assert call(s=7) == E              # shift >= window
    assert call(out=a) == E            # out overlaps x
    assert call(hd=64) == U
    assert call(M=4, H=16, W=16, s=0) == U    # windows of one token tile
    assert call(M=12, H=24, W=24, s=0) == U
    assert call(heads=8) == U          # C = 256 > 192
    assert call(B=0) == swa.SWIN_OK

