"""Pins for the oracle's MXFP4 decode and matrix-vector product.

Sources: "kimi-k3-in-c" README §4 (E2M1 table, E8M0 byte, nibble order, the
255 rule, the product over nibbles with one scale per 32-group)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_e2m1_table_matches_pages():
    table = _golden("e2m1_table.json")["values"]
    for code, v in enumerate(table):
        got = oracle.e2m1(code)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), code


def test_e8m0_all_bytes():
    for b in range(255):
        assert oracle.e8m0(b) == math.ldexp(1.0, b - 127), b
    assert oracle.e8m0(255) == 0.0
    # byte 0 is the subnormal 2^-127, not zero
    assert oracle.e8m0(0) > 0.0 and oracle.e8m0(0) == 2.0 ** -127


def test_expert_byte_census():
    g = _golden("e2m1_table.json")
    # 4 bits per weight plus one 8-bit scale per 32 weights
    assert 0.5 + 1.0 / g["group_size"] == g["bytes_per_weight"]
    assert g["expert_params"] * g["bytes_per_weight"] == g["expert_bytes"]
    # the pages' latent shape and the flat 7168 x 1536 shape hold the same bytes
    assert 3 * 3584 * 3072 == g["expert_params"] == 3 * 7168 * 1536


def _one_block(byte, scale, K=32):
    packed = np.zeros((1, K // 2), np.uint8)
    packed[0, 0] = byte
    scales = np.full((1, K // 32), scale, np.uint8)
    return packed, scales


@pytest.mark.parametrize("case", _golden("mxfp4_blocks.json")["cases"])
def test_hand_decoded_blocks(case):
    packed, scales = _one_block(case["byte"], case["scale"])
    even = oracle.mxfp4_gemv(np.eye(32)[0], packed, scales, 32, 1)[0]
    odd = oracle.mxfp4_gemv(np.eye(32)[1], packed, scales, 32, 1)[0]
    if "even" in case:
        assert even == case["even"] and odd == case["odd"]
        # a decoder with the nibbles swapped gives a different answer whenever
        # the two nibbles differ
        if case["even"] != case["odd"]:
            assert (even, odd) != (case["swapped_even"], case["swapped_odd"])
    else:
        assert even == 2.0 ** case["even_log2"] and odd == 2.0 ** case["odd_log2"]


def test_one_hot_columns_and_constant_rows():
    rng = np.random.default_rng(5)
    K, rows = 96, 5
    packed = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(110, 140, (rows, K // 32), dtype=np.uint8)
    table = _golden("e2m1_table.json")["values"]
    for c in (0, 1, 31, 32, 63, 94, 95):
        y = oracle.mxfp4_gemv(np.eye(K)[c], packed, scales, K, rows)
        for r in range(rows):
            b = int(packed[r, c // 2])
            code = (b >> 4) if (c & 1) else (b & 15)
            assert y[r] == table[code] * math.ldexp(1.0, int(scales[r, c // 32]) - 127)
    # constant code, constant scale, all-ones input: K * E2M1[c] * 2^(s-127)
    for code in range(16):
        byte = code | (code << 4)
        packed = np.full((1, K // 2), byte, np.uint8)
        scales = np.full((1, K // 32), 130, np.uint8)
        y = oracle.mxfp4_gemv(np.ones(K), packed, scales, K, 1)[0]
        assert y == K * table[code] * 8.0


def test_scale_255_drops_group_only():
    K = 64
    packed = np.full((1, K // 2), 0x22, np.uint8)  # every weight = 1.0
    scales = np.array([[255, 127]], np.uint8)
    y = oracle.mxfp4_gemv(np.ones(K), packed, scales, K, 1)[0]
    assert y == 32.0


def test_odd_width_tail_group():
    # a row whose width is not a multiple of 32 (the pages handle the tail)
    K = 37
    packed = np.full((1, (K + 1) // 2), 0x44, np.uint8)  # every weight = 2.0
    scales = np.array([[127, 128]], np.uint8)
    y = oracle.mxfp4_gemv(np.ones(K), packed, scales, K, 1)[0]
    assert y == 32 * 2.0 + 5 * 4.0


def _dense_decode(packed, scales, K):
    """Independent dense decode from the golden table (brute force)."""
    table = np.array(_golden("e2m1_table.json")["values"])
    rows = packed.shape[0]
    codes = np.empty((rows, K), np.int64)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    s = np.array([0.0 if b == 255 else math.ldexp(1.0, int(b) - 127) for b in range(256)])
    return table[codes] * np.repeat(s[scales], 32, axis=1)


def test_random_matches_dense_brute_force():
    rng = np.random.default_rng(11)
    K, rows = 256, 48
    packed = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(115, 135, (rows, K // 32), dtype=np.uint8)
    scales[3, 2] = 255
    scales[7, 0] = 0
    x = rng.standard_normal(K)
    W = _dense_decode(packed, scales, K)
    y, yabs = oracle.mxfp4_gemv(x, packed, scales, K, rows, want_abs=True)
    ref = W @ x
    refabs = np.abs(W) @ np.abs(x)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * refabs.max())
    np.testing.assert_allclose(yabs, refabs, rtol=1e-14)


def test_bf16_gemv_matches_numpy():
    import synth
    rng = np.random.default_rng(3)
    K, rows = 200, 9
    W = synth.bf16_bits(rng.standard_normal((rows, K)))
    x = rng.standard_normal(K)
    y, yabs = oracle.bf16_gemv(x, W, K, rows, want_abs=True)
    Wf = synth.bf16_to_f32(W).astype(np.float64)
    np.testing.assert_allclose(y, Wf @ x, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(yabs, np.abs(Wf) @ np.abs(x), rtol=1e-14)
    # bf16 widening is exact: a one-hot input returns the stored weight exactly
    y1 = oracle.bf16_gemv(np.eye(K)[17], W, K, rows)
    assert np.array_equal(y1, Wf[:, 17])
