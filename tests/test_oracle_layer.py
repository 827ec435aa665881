"""Pins for the oracle's whole layer on tiny shapes.

Source: "kimi-k3-in-c" README §9 (k3_moe: experts in router order, weighted
sum, shared expert added unweighted afterwards; dropped experts counted)."""
import json
import math
import os

import numpy as np

import oracle
import synth
from conftest import GOLDEN

TABLE = np.array(json.load(open(os.path.join(GOLDEN, "e2m1_table.json")))["values"])


def _dense(packed, scales):
    """Independent dense decode [rows][K] from the golden E2M1 table."""
    rows, half = packed.shape
    K = 2 * half
    codes = np.empty((rows, K), np.int64)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    s = np.array([0.0 if b == 255 else math.ldexp(1.0, b - 127) for b in range(256)])
    return TABLE[codes] * np.repeat(s[scales], 32, axis=1)


def _setup(spec, T, experts=None):
    E = spec.n_experts
    experts = list(range(E)) if experts is None else experts
    x = synth.make_x(spec, T)
    Wr = synth.make_router(spec)
    bias = synth.make_bias(spec)
    idx, w = oracle.route(x, Wr, bias, spec.topk)
    h = synth.expert_host(spec, experts)
    es = oracle.ExpertSet(experts, E, h["gate_packed"], h["gate_scales"], h["up_packed"],
                          h["up_scales"], h["down_packed"], h["down_scales"])
    return x, idx, w, h, es


def _act(g, u, spec):
    f = np.vectorize(lambda a, b: oracle.act(a, b, spec.act, spec.situ_b1, spec.situ_b2))
    return f(g, u)


def test_matches_dense_gated_sum():
    spec = synth.tiny_spec(seed=1)
    spec.bias_std = 0.05
    T = 4
    x, idx, w, h, es = _setup(spec, T)
    out, denom, drops = oracle.forward(x, idx, w, es, spec.hidden, spec.inter)
    assert drops == 0
    xf = synth.bf16_to_f32(x).astype(np.float64)
    for t in range(T):
        G = np.zeros(spec.n_experts)
        for j in range(spec.topk):
            G[idx[t, j]] = w[t, j]
        ref = np.zeros(spec.hidden)
        for e in range(spec.n_experts):   # every expert, gated (brute force)
            g = _dense(h["gate_packed"][e], h["gate_scales"][e]) @ xf[t]
            u = _dense(h["up_packed"][e], h["up_scales"][e]) @ xf[t]
            y = _dense(h["down_packed"][e], h["down_scales"][e]) @ _act(g, u, spec)
            ref += G[e] * y
        np.testing.assert_allclose(out[t], ref, rtol=0, atol=1e-12 * denom[t].max())
        assert np.all(np.abs(out[t]) <= denom[t] * (1 + 1e-12))


def test_unselected_experts_contribute_exactly_zero():
    spec = synth.tiny_spec(seed=2)
    T = 3
    x, idx, w, h, es = _setup(spec, T)
    out, _, _ = oracle.forward(x, idx, w, es, spec.hidden, spec.inter)
    used = set(idx.ravel().tolist())
    rng = np.random.default_rng(9)
    poisoned = {k: v.copy() for k, v in h.items()}
    for e in range(spec.n_experts):
        if e in used:
            continue
        for k in poisoned:
            if k.endswith("packed"):
                poisoned[k][e] = rng.integers(0, 256, poisoned[k][e].shape, dtype=np.uint8)
            else:
                poisoned[k][e] = 254
    es2 = oracle.ExpertSet(range(spec.n_experts), spec.n_experts, poisoned["gate_packed"],
                           poisoned["gate_scales"], poisoned["up_packed"], poisoned["up_scales"],
                           poisoned["down_packed"], poisoned["down_scales"])
    out2, _, _ = oracle.forward(x, idx, w, es2, spec.hidden, spec.inter)
    assert np.array_equal(out, out2)


def test_down_scale_plus_one_doubles_output():
    spec = synth.tiny_spec(seed=3)
    x, idx, w, h, es = _setup(spec, 2)
    out, _, _ = oracle.forward(x, idx, w, es, spec.hidden, spec.inter)
    ds = h["down_scales"].copy() + 1
    es2 = oracle.ExpertSet(range(spec.n_experts), spec.n_experts, h["gate_packed"], h["gate_scales"],
                           h["up_packed"], h["up_scales"], h["down_packed"], ds)
    out2, _, _ = oracle.forward(x, idx, w, es2, spec.hidden, spec.inter)
    assert np.array_equal(out2, 2.0 * out)


def test_relabelling_experts_is_invisible():
    spec = synth.tiny_spec(seed=4)
    spec.bias_std = 0.02
    T = 3
    x = synth.make_x(spec, T)
    Wr = synth.make_router(spec)
    bias = synth.make_bias(spec)
    h = synth.expert_host(spec, range(spec.n_experts))
    idx, w = oracle.route(x, Wr, bias, spec.topk)
    es = oracle.ExpertSet(range(spec.n_experts), spec.n_experts, h["gate_packed"], h["gate_scales"],
                          h["up_packed"], h["up_scales"], h["down_packed"], h["down_scales"])
    out, _, _ = oracle.forward(x, idx, w, es, spec.hidden, spec.inter)
    perm = np.random.default_rng(1).permutation(spec.n_experts)  # new id of old expert e = perm[e]
    inv = np.argsort(perm)
    idx2, w2 = oracle.route(x, Wr[inv], bias[inv], spec.topk)
    assert np.array_equal(idx2, perm[idx]) and np.array_equal(w2, w)
    es2 = oracle.ExpertSet(range(spec.n_experts), spec.n_experts,
                           *(h[k][inv] for k in ("gate_packed", "gate_scales", "up_packed",
                                                 "up_scales", "down_packed", "down_scales")))
    out2, _, _ = oracle.forward(x, idx2, w2, es2, spec.hidden, spec.inter)
    assert np.array_equal(out, out2)


def test_bad_indices_are_counted_drops():
    spec = synth.tiny_spec(seed=5)
    x, idx, w, h, es = _setup(spec, 2)
    bad = idx.copy()
    bad[0, 1] = -1
    bad[1, 0] = spec.n_experts
    out, _, drops = oracle.forward(x, bad, w, es, spec.hidden, spec.inter)
    assert drops == 2
    w0 = w.copy()
    w0[0, 1] = 0.0
    w0[1, 0] = 0.0
    ref, _, _ = oracle.forward(x, idx, w0, es, spec.hidden, spec.inter)
    np.testing.assert_array_equal(out, ref)


def test_shared_expert_added_unweighted_after_routed_sum():
    spec = synth.LayerSpec(hidden=256, inter=128, n_experts=8, topk=2, shared_inter=96, seed=6)
    T = 2
    x, idx, w, h, es = _setup(spec, T)
    S = synth.make_shared(spec)
    out_s, den_s, _ = oracle.forward(x, idx, w, es, spec.hidden, spec.inter, shared=S)
    out_r, den_r, _ = oracle.forward(x, idx, w, es, spec.hidden, spec.inter)
    # scaling every routing weight by zero leaves exactly the shared expert
    out_0, _, _ = oracle.forward(x, idx, 0 * w, es, spec.hidden, spec.inter, shared=S)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    S1, S3, S2 = (synth.bf16_to_f32(s).astype(np.float64) for s in S)
    for t in range(T):
        a = _act(S1 @ xf[t], S3 @ xf[t], spec)
        ref = S2 @ a
        np.testing.assert_allclose(out_0[t], ref, rtol=0, atol=1e-12 * (np.abs(S2) @ np.abs(a)).max())
        np.testing.assert_allclose(out_s[t] - out_r[t], ref, rtol=0, atol=1e-12 * den_s[t].max())
        assert np.all(den_s[t] >= den_r[t])


def test_swiglu_layer_matches_dense():
    spec = synth.tiny_spec(seed=7)
    spec.act = oracle.ACT_SWIGLU
    x, idx, w, h, es = _setup(spec, 2)
    out, denom, _ = oracle.forward(x, idx, w, es, spec.hidden, spec.inter, act_kind=oracle.ACT_SWIGLU)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    import torch
    for t in range(2):
        ref = np.zeros(spec.hidden)
        for j in range(spec.topk):
            e = idx[t, j]
            g = _dense(h["gate_packed"][e], h["gate_scales"][e]) @ xf[t]
            u = _dense(h["up_packed"][e], h["up_scales"][e]) @ xf[t]
            a = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
            ref += w[t, j] * (_dense(h["down_packed"][e], h["down_scales"][e]) @ a)
        np.testing.assert_allclose(out[t], ref, rtol=0, atol=1e-12 * denom[t].max())
