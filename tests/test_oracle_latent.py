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
