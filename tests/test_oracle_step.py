"""Pins of the oracle's pre-MoE norm (the decoder-layer listing: the MoE reads
k3_rmsnorm of the residual stream with the post-attention gain; README §5,
k3_rmsnorm, in its float form) and of its bf16 rounding, against values fixed
by IEEE arithmetic and closed forms, not by the oracle's own formula."""
import math

import numpy as np

import oracle


def _bits(v):
    return int(np.float32(v).view(np.uint32))


def test_bf16_round_to_nearest_even():
    # textbook cases: exact, ties to even both ways, just above a tie,
    # negative tie, 0.1 (0x3DCCCCCD rounds up), pi (0x40490FDB rounds down),
    # an fp32 subnormal-range exponent with an exact bf16 value
    cases = [(1.0, 0x3F80), (1 + 2 ** -8, 0x3F80), (1 + 3 * 2 ** -8, 0x3F82),
             (1 + 2 ** -8 + 2 ** -20, 0x3F81), (-(1 + 2 ** -8), 0xBF80),
             (0.1, 0x3DCD), (math.pi, 0x4049), (1.5 * 2.0 ** -126, 0x00C0),
             (0.0, 0x0000), (-2.5, 0xC020)]
    for v, want in cases:
        assert oracle.bf16_rne(v) == want, (v, hex(oracle.bf16_rne(v)), hex(want))


def test_bf16_rne_is_within_half_a_step_and_keeps_exact_values():
    rng = np.random.default_rng(3)
    for v in rng.standard_normal(2000).astype(np.float32) * 37:
        b = oracle.bf16_rne(v)
        back = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        step = 2.0 ** (math.floor(math.log2(abs(float(v)))) - 7)
        assert abs(back - float(v)) <= step / 2
        assert oracle.bf16_rne(back) == b   # a bf16 value is its own rounding


def test_unit_rms_input_is_the_gain_rounded():
    # all-ones rows have mean square 1; with a negligible eps inv is exactly 1
    # and each token element is bf16(gamma_i)
    h = np.ones((2, 8), np.float32)
    g = np.array([1, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 0.1, -2.5, 1, 0.5, 3], np.float32)
    x = oracle.prenorm_bf16(h, g, 1e-30)
    want = [0x3F80, 0x3F80, 0x3F82, 0x3DCD, 0xC020, 0x3F80, 0x3F00, 0x4040]
    assert x[0].tolist() == want and x[1].tolist() == want


def test_eps_sits_inside_the_root():
    # h = 0.1 everywhere, eps = 0.01: inside the root 0.1 / sqrt(0.01 + 0.01)
    # = 1/sqrt(2) -> bf16 0x3F35; eps added outside would give 0.1/0.11 = 0.909
    h = np.full((1, 64), 0.1, np.float32)
    x = oracle.prenorm_bf16(h, np.ones(64, np.float32), 0.01)
    assert set(x[0].tolist()) == {0x3F35}
    val = float(np.array([0x3F35 << 16], np.uint32).view(np.float32)[0])
    assert abs(val - 1 / math.sqrt(2)) <= 2 ** -9


def test_power_of_two_scaling_of_the_stream_changes_nothing():
    # scaling h by 2^k scales the fp64 sum of squares by 4^k exactly, so inv
    # by 2^-k exactly (eps negligible): h * inv is bit-identical
    rng = np.random.default_rng(5)
    h = rng.standard_normal((4, 512)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(512)).astype(np.float32)
    x0 = oracle.prenorm_bf16(h, g, 1e-30)
    for k in (-3, 5, 11):
        assert np.array_equal(oracle.prenorm_bf16(h * np.float32(2.0 ** k), g, 1e-30), x0)


def test_normed_tokens_have_unit_rms_and_power_of_two_gains_shift_exponents():
    rng = np.random.default_rng(6)
    h = (rng.standard_normal((3, 1024)) * 7).astype(np.float32)
    x = oracle.prenorm_bf16(h, np.ones(1024, np.float32), 1e-5)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rms = np.sqrt((xv ** 2).mean(axis=1))
    ms = (h.astype(np.float64) ** 2).mean(axis=1)
    np.testing.assert_allclose(rms, 1 / np.sqrt(1 + 1e-5 / ms), rtol=2 ** -8)
    # a gain of 2^k on one element moves only that element's exponent by k
    g = np.ones(1024, np.float32)
    g[::3] = 4.0
    x4 = oracle.prenorm_bf16(h, g, 1e-5)
    sel = np.zeros(1024, bool)
    sel[::3] = True
    nz = (x[:, sel] & 0x7FFF) != 0
    assert np.array_equal((x4[:, sel].astype(np.int32) - x[:, sel])[nz], np.full(nz.sum(), 2 << 7))
    assert np.array_equal(x4[:, ~sel], x[:, ~sel])


def test_sign_of_the_stream_flips_the_tokens():
    rng = np.random.default_rng(8)
    h = rng.standard_normal((2, 256)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(256)).astype(np.float32)
    a, b = oracle.prenorm_bf16(h, g, 1e-5), oracle.prenorm_bf16(-h, g, 1e-5)
    assert np.array_equal(a ^ b, np.full(a.shape, 0x8000, np.uint16))
