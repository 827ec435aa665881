"""GPU parity of k3moe_step: the decoder layer's pre-MoE norm of the fp32
residual stream (k3_rmsnorm's float form, rounded to the layer's bf16
tokens), routing, the expert layer, and the residual add, through the C ABI,
against the oracle.

Bars: the normed bf16 tokens bit-identical to the oracle's (on tokens whose
fp32 inv is not within the fp64 summation error of a rounding boundary; every
token here is); routes as in the layer tests; the updated stream within
1e-4 of D plus the one fp32 rounding of the add; the bf16 copy equal to the
round-to-nearest-even of the GPU's own fp32 value. Every input is seeded and
synthetic; expected values come only from ``oracle``."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (_REDRAW, _REDRAW_MAX, REL_TOL, bf16_rne_np, check_route, oracle_forward,
                         route_certificate)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EPS = 1e-5


def _layer(spec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import synth.device as sd
    t = sd.layer_tensors(spec, 0, DEV)
    return t, sd.make_layer(spec, t)


def _inv_certified(h, eps):
    """Per row: the exact fp64 value of 1/sqrt(mean(h^2) + eps) is farther
    from an fp32 rounding boundary than any fp64 summation order can move it."""
    T, n = h.shape
    ok = np.zeros(T, bool)
    for t in range(T):
        ss = math.fsum(float(v) * float(v) for v in h[t].astype(np.float64))
        y = 1.0 / math.sqrt(ss / n + float(np.float32(eps)))
        f = np.float32(y)
        lo = float(np.nextafter(f, np.float32(0)))
        hi = float(np.nextafter(f, np.float32(np.inf)))
        mids = ((float(f) + lo) / 2, (float(f) + hi) / 2)
        ok[t] = all(abs(y - m) > 1e-11 * y for m in mids)
    return ok


def _certified_stream(spec, T, scale, attempt, gamma_np):
    """A residual stream whose normed tokens all have certified routes: row t
    of an uncertified token is redrawn as the single row
    make_residual(spec, 1, attempt=_REDRAW + 64 t + a) for the next a."""
    h_np = synth.make_residual(spec, T, scale=scale, attempt=attempt)
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    for a in range(_REDRAW_MAX):
        x_ref = oracle.prenorm_bf16(h_np, gamma_np, EPS)
        _, _, _, ch = oracle.route(x_ref, Wr, bias, spec.topk, renorm=spec.renorm,
                                   routed_scale=spec.routed_scale, want_detail=True)
        bad = np.nonzero(~route_certificate(ch, spec.topk))[0]
        if bad.size == 0:
            return h_np
        for t in bad:
            h_np[t] = synth.make_residual(spec, 1, scale=scale, attempt=_REDRAW + int(t) * _REDRAW_MAX + a)[0]
    raise AssertionError("a token stayed uncertified")


def _step(spec, layer, T, scale=4.0, tokens=None, with_outputs=True, attempt=0):
    gamma_np = synth.make_post_norm(spec)
    h_np = _certified_stream(spec, T, scale, attempt, gamma_np)
    h = torch.from_numpy(h_np).to(DEV)
    gamma = torch.from_numpy(gamma_np).to(DEV)
    idx = torch.empty((T, spec.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((T, spec.topk), dtype=torch.float32, device=DEV)
    x = torch.empty((T, spec.hidden), dtype=torch.int16, device=DEV) if with_outputs else None
    hb = torch.empty((T, spec.hidden), dtype=torch.int16, device=DEV) if with_outputs else None
    print(f"[step] hidden={spec.hidden} latent={spec.latent} T={T}", flush=True)
    layer.step(h, gamma, EPS, idx, w, x_out=x, hb=hb)
    torch.cuda.synchronize()
    h_new = h.cpu().numpy()
    idx_g, w_g = idx.cpu().numpy(), w.cpu().numpy()

    x_ref = oracle.prenorm_bf16(h_np, gamma_np, EPS)
    assert _inv_certified(h_np, EPS).all()
    if with_outputs:
        assert np.array_equal(x.cpu().numpy().view(np.uint16), x_ref)
        assert np.array_equal(hb.cpu().numpy().view(np.uint16), bf16_rne_np(h_new))
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    idx_r, w_r, _, ch = oracle.route(x_ref[tokens], synth.make_router(spec), synth.make_bias(spec),
                                     spec.topk, renorm=spec.renorm, routed_scale=spec.routed_scale,
                                     want_detail=True)
    assert check_route(idx_g[tokens], w_g[tokens], idx_r, w_r, ch, spec.topk) == tokens.size
    # the layer output for the GPU's own routes, added to the stream
    ref, denom, drops = oracle_forward(spec, x_ref, idx_g, w_g, tokens=tokens)
    assert drops == 0
    want = h_np[tokens].astype(np.float64) + ref
    bound = REL_TOL * denom * (1 + 2.0 ** -24) + 2.0 ** -24 * np.abs(want)
    ratio = float((np.abs(h_new[tokens].astype(np.float64) - want) / bound).max())
    print(f"[step] T={T} max err / bound {ratio:.3g}", flush=True)
    assert ratio <= 1.0
    return h_new, idx_g


@pytest.mark.parametrize("T", [1, 3, 17, 40])
def test_tiny_step(T):
    spec = synth.LayerSpec(hidden=256, inter=128, n_experts=8, topk=2, shared_inter=128,
                           bias_std=0.05, seed=120 + T)
    _, layer = _layer(spec)
    _step(spec, layer, T)


def test_step_without_optional_outputs_gives_the_same_stream():
    spec = synth.LayerSpec(hidden=512, inter=256, n_experts=16, topk=4, shared_inter=256,
                           bias_std=0.05, seed=131)
    _, layer = _layer(spec)
    a, _ = _step(spec, layer, 9)
    b, _ = _step(spec, layer, 9, with_outputs=False)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T", [1, 5, 40])
def test_mid_latent_step(T):
    spec = synth.LayerSpec(hidden=1024, inter=512, n_experts=16, topk=4, shared_inter=512,
                           bias_std=0.05, seed=140 + T, latent=512)
    _, layer = _layer(spec)
    _step(spec, layer, T)


@pytest.mark.parametrize("hidden", [8192, 8704])
def test_wide_row_step(hidden):
    # rows up to 8192 are normed from registers in one read, wider ones in two
    # passes over the row
    spec = synth.LayerSpec(hidden=hidden, inter=128, n_experts=8, topk=2, shared_inter=128,
                           bias_std=0.05, seed=160 + hidden % 7)
    _, layer = _layer(spec)
    _step(spec, layer, 3)


def test_step_refusals():
    import mxfp4_routed_expert_sigmoid_amd as k3
    spec = synth.LayerSpec(hidden=256, inter=128, n_experts=8, topk=2, shared_inter=0,
                           bias_std=0.05, seed=150)
    _, layer = _layer(spec)
    h = torch.zeros((2, 256), dtype=torch.float32, device=DEV)
    g = torch.ones(256, dtype=torch.float32, device=DEV)
    idx = torch.empty((2, 2), dtype=torch.int32, device=DEV)
    w = torch.empty((2, 2), dtype=torch.float32, device=DEV)
    for eps in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(k3.K3MoeError):
            layer.step(h, g, eps, idx, w)
    with pytest.raises(k3.K3MoeError):   # h not 16-byte aligned
        layer.step(torch.zeros(2 * 256 + 1, dtype=torch.float32, device=DEV)[1:].view(2, 256), g, EPS, idx, w)
    # T = 0: nothing happens
    layer.step(h[:0], g, EPS, idx[:0], w[:0])
    torch.cuda.synchronize()


_FULL = {}


def _full():
    if "flat" not in _FULL:
        spec = synth.full_spec(seed=0)
        _FULL["flat"] = (spec,) + _layer(spec)
    return _FULL["flat"]


def test_full_step_T1():
    spec, _, layer = _full()
    a, idx = _step(spec, layer, 1)
    b, _ = _step(spec, layer, 1)
    assert np.array_equal(a, b)   # bitwise reproducible


def test_full_step_T64_sampled():
    spec, _, layer = _full()
    _step(spec, layer, 64, tokens=np.arange(0, 64, 4))
    _FULL.clear()


@pytest.mark.parametrize("T,latent", [(1, 0), (5, 0), (1, 512), (5, 512)])
def test_forward_residual_is_forward_plus_the_stream(T, latent):
    # h += forward(x) fused into the last kernel: bit-identical to forward
    # followed by one fp32 add; the bf16 copy is the nearest-even rounding;
    # writing the copy over x itself gives the same bits
    import synth.device as sd
    spec = synth.LayerSpec(hidden=1024, inter=512, n_experts=16, topk=4, shared_inter=512,
                           bias_std=0.05, seed=160 + T, latent=latent)
    _, layer = _layer(spec)
    x_np = synth.make_x(spec, T)
    x = sd.bf16_tensor(x_np, DEV)
    idx = torch.empty((T, spec.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((T, spec.topk), dtype=torch.float32, device=DEV)
    layer.route(x, idx, w)
    out = torch.empty((T, spec.hidden), dtype=torch.float32, device=DEV)
    layer.forward(x, idx, w, out)
    h0 = synth.make_residual(spec, T)
    h = torch.from_numpy(h0).to(DEV)
    hb = torch.empty((T, spec.hidden), dtype=torch.int16, device=DEV)
    layer.forward_residual(x, idx, w, h, hb=hb)
    h2 = torch.from_numpy(h0).to(DEV)
    x2 = x.clone()
    layer.forward_residual(x2, idx, w, h2, hb=x2)
    torch.cuda.synchronize()
    want = (h0 + out.cpu().numpy()).astype(np.float32)
    assert np.array_equal(h.cpu().numpy(), want)
    assert np.array_equal(hb.cpu().numpy().view(np.uint16), bf16_rne_np(want))
    assert np.array_equal(h2.cpu().numpy(), want)
    assert np.array_equal(x2.view(torch.int16).cpu().numpy().view(np.uint16), bf16_rne_np(want))
