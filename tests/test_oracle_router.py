"""Pins for the oracle's router.

Source: "kimi-k3-in-c" README §9 "Picking 16 experts of 896" (k3_router) and
the "Three invariants" section (the bias steers selection only)."""
import json
import math
import os

import numpy as np

import oracle
import synth
from conftest import GOLDEN

FIX = json.load(open(os.path.join(GOLDEN, "router_fixture.json")))


def _fixture_inputs():
    H, E = 32, 4
    rows = FIX["rows"]
    x = np.zeros((len(rows), H), np.float64)
    for t, r in enumerate(rows):
        x[t, :E] = r["logits"]
    Wr = np.zeros((E, H))
    Wr[np.arange(E), np.arange(E)] = 1.0
    xb, Wb = synth.bf16_bits(x), synth.bf16_bits(Wr)
    assert np.array_equal(synth.bf16_to_f32(xb), x.astype(np.float32))  # bf16-exact
    return xb, Wb


def _sig(v):
    return 1.0 / (1.0 + math.exp(-v))


def test_bias_fixture_reorders_five_of_six():
    x, Wr = _fixture_inputs()
    bias = np.array(FIX["bias"], np.float32)
    idx_b, w_b = oracle.route(x, Wr, bias, FIX["topk"])
    idx_u, w_u = oracle.route(x, Wr, None, FIX["topk"])
    changed = 0
    for t, r in enumerate(FIX["rows"]):
        assert list(idx_b[t]) == r["biased_top2"], t
        assert list(idx_u[t]) == r["unbiased_top2"], t
        changed += list(idx_b[t]) != list(idx_u[t])
    assert changed == FIX["rows_reordered_by_bias"]


def test_weights_come_from_unbiased_scores():
    x, Wr = _fixture_inputs()
    bias = np.array(FIX["bias"], np.float32)
    idx, w = oracle.route(x, Wr, bias, FIX["topk"])
    for t, r in enumerate(FIX["rows"]):
        i0, i1 = idx[t]
        s0, s1 = _sig(r["logits"][i0]), _sig(r["logits"][i1])
        # renormalised unbiased scores
        assert abs(w[t, 0] - s0 / (s0 + s1)) < 2e-7 and abs(w[t, 1] - s1 / (s0 + s1)) < 2e-7
        # and not the biased ones (which differ by more than float noise here)
        c0, c1 = s0 + FIX["bias"][i0], s1 + FIX["bias"][i1]
        if FIX["bias"][i0] != FIX["bias"][i1]:
            assert abs(w[t, 0] - c0 / (c0 + c1)) > 1e-4


def test_no_renorm_and_routed_scale():
    x, Wr = _fixture_inputs()
    idx, w = oracle.route(x, Wr, None, 2, renorm=0, routed_scale=2.5)
    for t, r in enumerate(FIX["rows"]):
        for j in range(2):
            sc = np.float32(_sig(r["logits"][idx[t, j]]))
            assert w[t, j] == np.float32(sc * np.float32(2.5))
    idx, w = oracle.route(x, Wr, None, 2, renorm=1, routed_scale=2.5)
    np.testing.assert_allclose(w.sum(axis=1), 2.5, rtol=1e-6)


def test_unbiased_topk_is_argsort_of_logits():
    spec = synth.LayerSpec(hidden=512, inter=64, n_experts=64, topk=6, seed=4)
    x = synth.make_x(spec, 7)
    Wr = synth.make_router(spec)
    idx, w, logits, ch = oracle.route(x, Wr, None, spec.topk, want_detail=True)
    # library reference: numpy matmul of the widened bf16 values, then a sort
    L = synth.bf16_to_f32(x).astype(np.float64) @ synth.bf16_to_f32(Wr).astype(np.float64).T
    np.testing.assert_allclose(logits, L, rtol=1e-12, atol=1e-12)
    for t in range(x.shape[0]):
        order = np.lexsort((np.arange(spec.n_experts), -L[t]))[: spec.topk]
        assert list(idx[t]) == list(order)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)


def test_ties_go_to_lowest_index():
    H, E = 32, 8
    Wr = np.zeros((E, H))
    Wr[:, 0] = [0.5, 1.0, 2.0, 0.25, 1.0, 2.0, 0.0, 2.0]
    x = np.zeros((1, H))
    x[0, 0] = 1.0
    idx, w = oracle.route(synth.bf16_bits(x), synth.bf16_bits(Wr), None, 5)
    assert list(idx[0]) == [2, 5, 7, 1, 4]
