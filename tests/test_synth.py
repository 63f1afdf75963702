"""The seeded input generator: reproducible, prefix-stable, and its bfloat16
rounding agrees with torch's round-to-nearest-even conversion."""
import numpy as np
import torch

import synth


def test_splitmix64_reference_values():
    # SplitMix64 seeded with 1234567: the first outputs of the published
    # generator (state += golden gamma; mix with the 30/27/31 shifts)
    z = synth.splitmix64(1234567, 0, 3)
    assert z.tolist() == [6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_counter_form_slices_agree():
    key = synth.stream_key(1004, 0)
    full = synth.splitmix64(key, 0, 1000)
    assert np.array_equal(full[300:700], synth.splitmix64(key, 300, 400))


def test_normal_moments_and_prefix():
    x = synth.normal(synth.stream_key(7, 0), 1 << 20)
    assert abs(float(x.mean())) < 5e-3 and abs(float(x.std()) - 1.0) < 5e-3
    assert np.array_equal(synth.normal(synth.stream_key(7, 0), 1001), x[:1001])


def test_bf16_rounding_matches_torch():
    x = synth.normal(synth.stream_key(3, 0), 1 << 16, 3.0)
    x = np.concatenate([x, np.array([0.0, -0.0, 1.0, 65504.0, 1e-30, -3.3895314e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_bits(x), ref)
    assert np.array_equal(synth.bf16_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_smaller_batch_is_a_prefix():
    a, ta = synth.workload_inputs("swin-t-s3", batch=2)
    b, tb = synth.make_inputs(3, 14, 14, 12, 32, 7, seed=1003)
    assert np.array_equal(a, b[:2]) and np.array_equal(ta, tb)


def test_linear_inputs_prefix_and_shapes():
    for name, w in synth.LINEAR_WORKLOADS.items():
        x, wt, b, r = synth.linear_inputs(name, tokens=5)
        x2, wt2, b2, r2 = synth.linear_inputs(name, tokens=9)
        assert x.shape == (5, w["K"]) and wt.shape == (w["N"], w["K"]) and b.shape == (w["N"],)
        assert x.dtype == np.uint16 and wt.dtype == np.uint16 and b.dtype == np.float32
        assert np.array_equal(x, x2[:5]) and np.array_equal(wt, wt2) and np.array_equal(b, b2)
        assert (r is None) == (not w["residual"])
        if r is not None:
            assert r.shape == (5, w["N"]) and np.array_equal(r, r2[:5])


def test_ln_linear_inputs_prefix_and_shapes():
    for name, w in synth.LN_LINEAR_WORKLOADS.items():
        x, g, b, wt, bias = synth.ln_linear_inputs(name, tokens=4)
        x2, g2, _, wt2, _ = synth.ln_linear_inputs(name, tokens=7)
        assert x.shape == (4, w["K"]) and g.shape == (w["K"],) and wt.shape == (w["N"], w["K"])
        assert g.dtype == np.float32 and bias.shape == (w["N"],)
        assert np.array_equal(x, x2[:4]) and np.array_equal(g, g2) and np.array_equal(wt, wt2)


def test_int8_codes_range_and_prefix():
    key = synth.stream_key(5, 10)
    c = synth.int8_codes(key, 100000)
    assert c.dtype == np.int8 and c.min() >= -127 and c.max() <= 127
    assert 31.0 < c.astype(np.float64).std() < 33.0
    assert np.array_equal(synth.int8_codes(key, 1000), c[:1000])
    codes, scales, table = synth.i8_inputs("swin-t-s3-i8", batch=2)
    assert codes.shape == (2, 14, 14, 3, 12, 32) and scales.dtype == np.float32
    assert np.array_equal(table, synth.workload_inputs("swin-t-s3", batch=1)[1])
