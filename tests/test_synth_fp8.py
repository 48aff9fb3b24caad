"""The host-side OCP e4m3 rounding that produces the fp8 inputs, checked
against an independent implementation (torch's float8_e4m3fn conversion) and
the format's defining values.  The oracle consumes the rounded values, so this
fixes what the fp8 parity tests compare against."""

import numpy as np
import torch

import synth


def test_fp8_rounding_matches_torch_and_format():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 4,
        np.array([0.0, -0.0, 448.0, -448.0, 2 ** -9, 2 ** -10, 3 * 2 ** -10, 1.0625, 1.1875, 0.9375, 15.5],
                 np.float32),
    ])
    b = synth.fp8_bits(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(b, want)
    v = synth.fp8_decode(b)
    np.testing.assert_array_equal(v, torch.from_numpy(want).view(torch.float8_e4m3fn).float().numpy())
    # format: 448 is the largest finite value (0x7E); the smallest subnormal is 2^-9
    assert synth.fp8_bits(np.float32([448.0]))[0] == 0x7E and synth.fp8_decode(np.uint8([0x01]))[0] == 2.0 ** -9
    # ties go to the even code: 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39)
    assert synth.fp8_bits(np.float32([1.0625]))[0] == 0x38
    # relative rounding error of normal values is at most 2^-4
    nz = np.abs(x) >= 2 ** -6
    assert np.max(np.abs(v[nz] - x[nz]) / np.abs(x[nz])) <= 2.0 ** -4


def test_fp8_layer_inputs_are_the_rounded_draws():
    spec = synth.config_layers(2, 30)[0]
    a = synth.make_tt_layer(2, 0, spec, 64, 0.4, "fp8")
    b = synth.make_tt_layer(2, 0, spec, 64, 0.4, "f32")
    assert a["x_bits"].dtype == np.uint8
    np.testing.assert_array_equal(a["x"], synth.fp8_decode(synth.fp8_bits(b["x"])))
