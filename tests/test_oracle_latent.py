"""Pins for the oracle's latent layer (the experts between a down- and an
up-projection, RMSNorm on the aggregate).

Source: "kimi-k3-in-c" README §9 (k3_moe, its six steps: route on the full
width, down-project into the latent, experts at the latent width summed in
router order, RMSNorm of the AGGREGATE, up-project, shared experts on the
ORIGINAL input added unweighted) and §5 (k3_rmsnorm: epsilon inside the
square root). Each pin ties the latent function to something fixed outside
it: the flat oracle (pinned in test_oracle_layer.py), closed forms of the
norm, or exact invariances."""
import numpy as np

import oracle
import synth


def _eye_bf16(n):
    return synth.bf16_bits(np.eye(n))


def _setup(spec, T, w_scale=1.0, bad=False):
    E = spec.n_experts
    x = synth.make_x(spec, T)
    idx, w = oracle.route(x, synth.make_router(spec), synth.make_bias(spec), spec.topk,
                          renorm=spec.renorm)
    w = (w * np.float32(w_scale)).astype(np.float32)
    if bad:
        idx = idx.copy()
        idx[0, 0] = -1
    h = synth.expert_host(spec, list(range(E)))
    es = oracle.ExpertSet(list(range(E)), E, h["gate_packed"], h["gate_scales"], h["up_packed"],
                          h["up_scales"], h["down_packed"], h["down_scales"])
    return x, idx, w, es


def _spec(**kw):
    d = dict(hidden=256, inter=128, n_experts=8, topk=2, shared_inter=0, seed=3, bias_std=0.05)
    d.update(kw)
    return synth.LayerSpec(**d)


def test_rmsnorm_closed_forms():
    out, inv = oracle.rmsnorm(np.array([3.0, 4.0]), None, 0.0)
    assert inv == 1.0 / np.sqrt(12.5)
    assert np.allclose(out, [3.0 * inv, 4.0 * inv], rtol=0, atol=0)
    # epsilon inside the root: mean square 12.5, eps 12.5 -> inv = 1/5
    _, inv = oracle.rmsnorm(np.array([3.0, 4.0]), None, 12.5)
    assert inv == 0.2
    out, _ = oracle.rmsnorm(np.array([3.0, 4.0]), np.array([2.0, -0.5], np.float32), 12.5)
    assert np.allclose(out, [1.2, -0.4], rtol=1e-15, atol=0)


def test_identity_projections_without_norm_equal_the_flat_layer():
    # L = H, down = up = identity, no norm: the latent layer is the flat one,
    # bit for bit (one exact product per projection output)
    spec = _spec(shared_inter=128, latent=256)
    x, idx, w, es = _setup(spec, 5)
    S = synth.make_shared(spec)
    I_ = _eye_bf16(256)
    lat, dl, _ = oracle.forward_latent(x, idx, w, es, 256, 256, 128, I_, I_, norm=False, shared=S)
    flat, df, _ = oracle.forward(x, idx, w, es, 256, 128, shared=S)
    assert np.array_equal(lat, flat)
    assert np.array_equal(dl, df)


def test_norm_is_on_the_aggregate_scale_invariance():
    # doubling every routing weight doubles the aggregate exactly; with eps 0
    # its RMSNorm is unchanged, so the output is bit-identical. (Norming each
    # expert and then summing would double the output instead.)
    spec = _spec(latent=128, renorm=0)
    x, idx, w, es = _setup(spec, 4)
    Wd, Wu, g = synth.make_latent(spec)
    a, _, _ = oracle.forward_latent(x, idx, w, es, 256, 128, 128, Wd, Wu, gamma=g, eps=0.0)
    b, _, _ = oracle.forward_latent(x, idx, 2 * w, es, 256, 128, 128, Wd, Wu, gamma=g, eps=0.0)
    assert np.array_equal(a, b)
    # a positive epsilon breaks the invariance (it is used)
    c, _, _ = oracle.forward_latent(x, idx, w, es, 256, 128, 128, Wd, Wu, gamma=g, eps=1e3)
    d, _, _ = oracle.forward_latent(x, idx, 2 * w, es, 256, 128, 128, Wd, Wu, gamma=g, eps=1e3)
    assert not np.allclose(c, d, rtol=1e-6)


def test_normed_aggregate_has_unit_rms_and_eps_sits_inside_the_root():
    # identity projections, gamma 1, no shared: out = RMSNorm(accL) where accL
    # is the flat layer's routed output
    spec = _spec(latent=256)
    x, idx, w, es = _setup(spec, 3)
    I_ = _eye_bf16(256)
    flat, _, _ = oracle.forward(x, idx, w, es, 256, 128)
    out0, _, _ = oracle.forward_latent(x, idx, w, es, 256, 256, 128, I_, I_, gamma=None, eps=0.0)
    assert np.allclose(np.mean(out0 ** 2, axis=1), 1.0, rtol=1e-12)
    ms = np.mean(flat ** 2, axis=1)
    for t in range(3):
        eps = float(ms[t])   # eps equal to the mean square: RMS of the output 1/sqrt(2)
        o, _, _ = oracle.forward_latent(x[t:t + 1], idx[t:t + 1], w[t:t + 1], es, 256, 256, 128,
                                        I_, I_, gamma=None, eps=eps)
        assert np.isclose(np.mean(o ** 2), 0.5, rtol=1e-12)


def test_gamma_multiplies_elementwise():
    spec = _spec(latent=256)
    x, idx, w, es = _setup(spec, 2)
    I_ = _eye_bf16(256)
    g = (1.0 + 0.25 * np.arange(256) / 256.0).astype(np.float32)
    a, _, _ = oracle.forward_latent(x, idx, w, es, 256, 256, 128, I_, I_, gamma=None, eps=1e-5)
    b, _, _ = oracle.forward_latent(x, idx, w, es, 256, 256, 128, I_, I_, gamma=g, eps=1e-5)
    assert np.allclose(b, a * g.astype(np.float64), rtol=1e-15, atol=0)


def test_shared_expert_reads_the_original_input():
    # down-projection zero: the experts see z = 0, act(0, .) = 0, the normed
    # aggregate is 0, and the output is the shared expert on x alone, equal to
    # the flat layer with every routing weight zero
    spec = _spec(latent=128, shared_inter=128)
    x, idx, w, es = _setup(spec, 3)
    S = synth.make_shared(spec)
    _, Wu, g = synth.make_latent(spec)
    Z = np.zeros((128, 256), np.uint16)
    lat, _, _ = oracle.forward_latent(x, idx, w, es, 256, 128, 128, Z, Wu, gamma=g, shared=S)
    es_flat = oracle.ExpertSet([], 8, np.zeros((0, 128, 128), np.uint8), np.zeros((0, 128, 8), np.uint8),
                               np.zeros((0, 128, 128), np.uint8), np.zeros((0, 128, 8), np.uint8),
                               np.zeros((0, 256, 64), np.uint8), np.zeros((0, 256, 4), np.uint8))
    only_shared, _, _ = oracle.forward(x, np.full_like(idx, -1), w, es_flat, 256, 128, shared=S)
    assert np.array_equal(lat, only_shared)


def test_drops_counted_and_denominator_bounds_the_output():
    spec = _spec(latent=128, shared_inter=128)
    x, idx, w, es = _setup(spec, 4, bad=True)
    Wd, Wu, g = synth.make_latent(spec)
    out, den, drops = oracle.forward_latent(x, idx, w, es, 256, 128, 128, Wd, Wu, gamma=g,
                                            shared=synth.make_shared(spec))
    assert drops == 1
    assert np.all(den >= np.abs(out))
    assert np.all(den > 0)


# ---------------------------------------------------------------------------
# A dense numpy statement of the latent layer, written from README §9 k3_moe
# steps 2-6 with its own MXFP4 decode (from the golden E2M1 table) and its
# own activation: a check of the oracle that shares none of its code.
import json
import math
import os

from conftest import GOLDEN

_TABLE = np.array(json.load(open(os.path.join(GOLDEN, "e2m1_table.json")))["values"])


def _dense(packed, scales):
    rows, half = packed.shape
    codes = np.empty((rows, 2 * half), np.int64)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    s = np.array([0.0 if b == 255 else math.ldexp(1.0, b - 127) for b in range(256)])
    return _TABLE[codes] * np.repeat(s[scales], 32, axis=1)


def _situ(g, u, b1=4.0, b2=25.0):
    return b1 * np.tanh(g / b1) / (1.0 + np.exp(-g)) * (b2 * np.tanh(u / b2))


def _dense_latent(x, idx, w, h, Wd, Wu, gamma, eps, S, perturb=None):
    """Per token: z = Wd x; acc = sum_j w_j W2_e act(W1_e z, W3_e z) in router
    order; acc <- RMSNorm(acc) * gamma; out = Wu acc + S2 act(S1 x, S3 x).
    perturb(t, j, y, yabs) may replace an expert's output (error-bound check)."""
    bf = lambda a: synth.bf16_to_f32(a).astype(np.float64)
    xf, Wdf, Wuf = bf(x), bf(Wd), bf(Wu)
    S1, S3, S2 = (bf(m) for m in S)
    out = np.zeros((x.shape[0], Wuf.shape[0]))
    for t in range(x.shape[0]):
        z = Wdf @ xf[t]
        acc = np.zeros(Wdf.shape[0])
        for j in range(idx.shape[1]):
            e = idx[t, j]
            g = _dense(h["gate_packed"][e], h["gate_scales"][e]) @ z
            u = _dense(h["up_packed"][e], h["up_scales"][e]) @ z
            a = _situ(g, u)
            D2 = _dense(h["down_packed"][e], h["down_scales"][e])
            y = D2 @ a
            if perturb is not None:
                y = perturb(t, j, y, np.abs(D2) @ np.abs(a))
            acc += np.float64(w[t, j]) * y
        acc = acc / np.sqrt(np.mean(acc ** 2) + eps) * gamma.astype(np.float64)
        out[t] = Wuf @ acc + S2 @ _situ(S1 @ xf[t], S3 @ xf[t])
    return out


def _general_latent_case():
    # L != H, general (random) projections, the norm on with a non-trivial
    # gain, a shared expert, a positive epsilon
    spec = _spec(hidden=256, latent=128, inter=96, n_experts=6, topk=3, shared_inter=64, seed=11)
    x, idx, w, es = _setup(spec, 3)
    h = synth.expert_host(spec, list(range(spec.n_experts)))
    Wd, Wu, g = synth.make_latent(spec)
    S = synth.make_shared(spec)
    return spec, x, idx, w, es, h, Wd, Wu, g, S


def test_latent_matches_dense_numpy_general_projections():
    spec, x, idx, w, es, h, Wd, Wu, g, S = _general_latent_case()
    assert Wd.shape == (128, 256) and Wu.shape == (256, 128)
    eps = 1e-5
    out, den, drops = oracle.forward_latent(x, idx, w, es, 256, 128, 96, Wd, Wu, gamma=g, eps=eps,
                                            shared=S)
    assert drops == 0
    ref = _dense_latent(x, idx, w, h, Wd, Wu, g, eps, S)
    assert np.all(np.abs(out - ref) <= 1e-11 * den)
    # the routed part matters: dropping one slot's weight changes the result
    w2 = w.copy()
    w2[:, 0] = 0.0
    ref2 = _dense_latent(x, idx, w2, h, Wd, Wu, g, eps, S)
    assert np.max(np.abs(ref2 - ref) / den) > 1e-3


def test_latent_denominator_bounds_first_order_error():
    # D is the error denominator: a relative perturbation of at most r in
    # every expert product (each y_j[l] moved by up to r * sum_n |W2[l][n] a[n]|)
    # moves each output by at most r * D, to first order (the norm included)
    spec, x, idx, w, es, h, Wd, Wu, g, S = _general_latent_case()
    eps = 1e-5
    out, den, _ = oracle.forward_latent(x, idx, w, es, 256, 128, 96, Wd, Wu, gamma=g, eps=eps, shared=S)
    base = _dense_latent(x, idx, w, h, Wd, Wu, g, eps, S)
    r = 1e-7
    worst = 0.0
    for trial in range(6):
        rng = np.random.default_rng(100 + trial)
        signs = {}

        def perturb(t, j, y, yabs):
            s = signs.setdefault((t, j), rng.choice([-1.0, 1.0], size=y.shape) if trial < 4
                                 else np.sign(y + 1e-300))
            return y + r * s * yabs
        moved = _dense_latent(x, idx, w, h, Wd, Wu, g, eps, S, perturb=perturb)
        ratio = np.abs(moved - base) / (r * den)
        worst = max(worst, float(ratio.max()))
    assert worst <= 1.0 + 1e-3
    # and D is not loose by orders of magnitude
    assert worst >= 1e-2
