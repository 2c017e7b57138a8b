"""The seeded input generator: bf16 rounding, determinism, part-addressable seeds."""

import numpy as np

from megatron_tensor_layer_amd import inputs as I


def test_round_to_bf16_nearest_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6... -> even mantissa (1 + 2^-6)
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -2.5, 3.0e38], np.float32)
    r = I.round_to_bf16(x)
    np.testing.assert_array_equal(r[:5], np.array([1.0, 1.0, 1 + 2**-6, 1 + 2**-7, -2.5], np.float32))
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    # against the exhaustive definition: nearest of the two bf16 neighbours
    rng = np.random.default_rng(0)
    v = rng.standard_normal(10000).astype(np.float32)
    rb = I.round_to_bf16(v)
    lo = (v.view(np.uint32) & 0xFFFF0000).view(np.float32)
    hi = ((v.view(np.uint32) & 0xFFFF0000) + 0x10000).astype(np.uint32).view(np.float32)
    dlo, dhi = np.abs(v.astype(np.float64) - lo), np.abs(hi.astype(np.float64) - v)
    expect = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi,
                      np.where((lo.view(np.uint32) >> 16) % 2 == 0, lo, hi)))
    np.testing.assert_array_equal(rb, expect)


def test_draws_are_deterministic_and_part_addressable():
    c = I.make_config("tiny", h=32, a=4, s=8, b=2, t=4, dtype="bf16")
    w1 = I.param_full(c, "Wq")
    w2 = I.param_full(c, "Wq")
    np.testing.assert_array_equal(w1, w2)
    assert w1.shape == (32, 32)
    np.testing.assert_array_equal(w1[:, 8:16], I.param_part(c, "Wq", 1))
    np.testing.assert_array_equal(I.param_full(c, "Wo")[16:24], I.param_part(c, "Wo", 2))
    np.testing.assert_array_equal(I.param_full(c, "bo"), I.param_part(c, "bo", 3))
    assert abs(float(np.std(I.param_full(c, "W1"))) - 0.02) < 0.003
    x = I.activation(c, "X")
    assert x.shape == (16, 32)
    np.testing.assert_array_equal(x, I.round_to_bf16(x))


def test_prefix_of_a_draw_is_the_shorter_draw():
    c = I.make_config("tiny", h=32, a=4, s=8, b=2, t=4, dtype="fp32")
    np.testing.assert_array_equal(I.activation(c, "X")[:6], I.activation(c, "X", tokens=6))


def test_layernorm_params_are_rounded_and_spread_around_one():
    c = I.make_config("ln", h=4096, a=32, s=16, b=1, t=8, dtype="bf16")
    ln = I.ln_params(c)
    for n in I.LN_NAMES:
        assert ln[n].shape == (4096,)
        np.testing.assert_array_equal(ln[n], I.round_to_bf16(ln[n]))
    assert abs(float(np.mean(ln["g1"])) - 1.0) < 0.01 and abs(float(np.std(ln["g1"])) - 0.1) < 0.01
    assert abs(float(np.std(ln["be2"])) - 0.02) < 0.003
    assert not np.array_equal(ln["g1"], ln["g2"])
