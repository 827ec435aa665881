"""GPU parity of the fused one-token path (k3moe_route_forward at T = 1:
router + shared gate/up, top-k + routed gate/up + shared down, routed down +
router-order sum), through the C ABI, against the fp64 oracle.

Every input is seeded and synthetic (``synth``); expected values come only
from ``oracle``."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import REL_TOL, W_RTOL_WAVE, check_route, oracle_forward, rel_err, route_certificate

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import synth.device as sd
    return sd


def _make(spec):
    sd = _sd()
    t = sd.layer_tensors(spec, 0, DEV)
    return t, sd.make_layer(spec, t)


def _rf(layer, x_np, logits=False):
    """route_forward on one token: idx, w, out (and fp32 logits)."""
    import synth.device as sd
    T = x_np.shape[0]
    x = sd.bf16_tensor(x_np, DEV)
    K, E, H = layer.cfg.topk, layer.cfg.n_experts, layer.cfg.hidden
    idx = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), float("nan"), dtype=torch.float32, device=DEV)
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV) if logits else None
    layer.route_forward(x, idx, w, out, logits=lg)
    torch.cuda.synchronize()
    return (x, idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy(),
            None if lg is None else lg.cpu().numpy())


def _route(layer, x):
    T = x.shape[0]
    K, E = layer.cfg.topk, layer.cfg.n_experts
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    layer.route(x, idx, w, logits=lg)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


def _certified(spec, attempt0=0):
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    for attempt in range(attempt0, attempt0 + 50):
        x = synth.make_x(spec, 1, attempt=attempt)
        idx, w, logits, ch = oracle.route(x, Wr, bias, spec.topk, renorm=spec.renorm,
                                          routed_scale=spec.routed_scale, want_detail=True)
        if route_certificate(ch, spec.topk).all():
            return x, idx, w, logits, ch
    raise AssertionError("no certified token")


def _check_token(spec, layer, x_np, idx_r, w_r, ch):
    x, idx, w, out, lg = _rf(layer, x_np, logits=True)
    check_route(idx, w, idx_r, w_r, ch, spec.topk, w_rtol=W_RTOL_WAVE)
    assert np.array_equal(idx, idx_r)                      # certified: exact
    # the same router arithmetic as k3moe_route: identical ids, weights, logits
    i2, w2, lg2 = _route(layer, x)
    assert np.array_equal(i2, idx) and np.array_equal(w2, w) and np.array_equal(lg2, lg)
    ref, denom, drops = oracle_forward(spec, x_np, idx_r, w_r)
    assert drops == 0 and layer.error_count() == 0
    err = rel_err(out, ref, denom)
    assert err <= REL_TOL, err
    return x, out, err


_FULL = {}


def _full():
    if "f" not in _FULL:
        spec = synth.full_spec(seed=0)
        _FULL["f"] = (spec,) + _make(spec)
    return _FULL["f"]


@pytest.mark.parametrize("attempt", [0, 10, 20, 30])
def test_full_decode_fused_all_outputs(attempt):
    # the measured configuration: every one of the 7168 outputs of a token
    spec, t, layer = _full()
    x_np, idx_r, w_r, logits, ch = _certified(spec, attempt)
    x, out, _ = _check_token(spec, layer, x_np, idx_r, w_r, ch)
    # bitwise reproducible
    _, _, _, out2, _ = _rf(layer, x_np)
    assert np.array_equal(out, out2)


def test_full_decode_fused_agrees_with_forward():
    # the fused kernels and k3moe_forward on the same routes: both within the
    # bound of the oracle, and close to each other (another summation order)
    spec, t, layer = _full()
    x_np, idx_r, w_r, logits, ch = _certified(spec, 40)
    x, idx, w, out, _ = _rf(layer, x_np)
    o2 = torch.empty((1, spec.hidden), dtype=torch.float32, device=DEV)
    layer.forward(x, torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV), o2)
    torch.cuda.synchronize()
    ref, denom, _ = oracle_forward(spec, x_np, idx_r, w_r)
    assert rel_err(o2.cpu().numpy(), ref, denom) <= REL_TOL
    assert np.max(np.abs(out - o2.cpu().numpy()) / denom) <= 2 * REL_TOL


def test_full_decode_fused_poisoned_unselected_experts():
    # unselected experts contribute exactly zero: rewriting every other
    # expert's bytes (scale byte 254, random nibbles) leaves the output
    # bit-identical
    spec, t, layer = _full()
    x_np, idx_r, w_r, logits, ch = _certified(spec, 50)
    _, idx, _, out, _ = _rf(layer, x_np)
    used = set(idx.ravel().tolist())
    others = torch.tensor([e for e in range(spec.n_experts) if e not in used][:64], device=DEV)
    saved = {k: t[k][others].clone() for k in ("gate_packed", "gate_scales", "up_packed", "up_scales",
                                               "down_packed", "down_scales")}
    g = torch.Generator(device=DEV).manual_seed(5)
    for k in saved:
        if k.endswith("scales"):
            t[k][others] = 254
        else:
            t[k][others] = torch.randint(0, 256, t[k][others].shape, generator=g, device=DEV,
                                         dtype=torch.int32).to(torch.uint8)
    try:
        _, idx2, _, out2, _ = _rf(layer, x_np)
        assert np.array_equal(idx2, idx)
        assert np.array_equal(out2, out)
    finally:
        for k, v in saved.items():
            t[k][others] = v
        torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["mid", "mid_swiglu", "wide_e", "no_shared", "h3584"])
def test_fused_shapes(kind):
    # smaller layers through the same kernels: top-k in its own launch
    # (E <= 512) and inside the gate/up kernel (512 < E <= 1024), SwiGLU
    # without renormalisation, no shared expert, a 3584-wide token
    base = dict(bias_std=0.05)
    if kind == "mid":
        spec = synth.LayerSpec(hidden=512, inter=512, n_experts=16, topk=4, shared_inter=256, seed=81, **base)
    elif kind == "mid_swiglu":
        spec = synth.LayerSpec(hidden=512, inter=512, n_experts=16, topk=4, shared_inter=256, seed=82,
                               act=oracle.ACT_SWIGLU, renorm=0, routed_scale=2.5, **base)
    elif kind == "wide_e":
        spec = synth.LayerSpec(hidden=1024, inter=256, n_experts=640, topk=8, shared_inter=512, seed=83, **base)
    elif kind == "no_shared":
        spec = synth.LayerSpec(hidden=2048, inter=384, n_experts=600, topk=16, shared_inter=0, seed=84, **base)
    else:
        spec = synth.LayerSpec(hidden=3584, inter=2048, n_experts=8, topk=3, shared_inter=3072, seed=85, **base)
    t, layer = _make(spec)
    for attempt in (0, 7):
        x_np, idx_r, w_r, logits, ch = _certified(spec, attempt)
        _check_token(spec, layer, x_np, idx_r, w_r, ch)


def test_fused_scale_edge_bytes():
    # E8M0 byte 255 drops its group, byte 0 is 2^-127 and must not flush,
    # in every expert matrix, through the fused kernels
    spec = synth.LayerSpec(hidden=1024, inter=256, n_experts=16, topk=4, shared_inter=256, seed=86,
                           bias_std=0.05)
    t, layer = _make(spec)
    g = torch.Generator().manual_seed(3)
    for name in ("gate_scales", "up_scales", "down_scales"):
        s = t[name]
        m = torch.rand(s.shape, generator=g) < 0.05
        z = torch.rand(s.shape, generator=g) < 0.03
        s[m.to(DEV)] = 255
        s[z.to(DEV)] = 0
    torch.cuda.synchronize()
    host = {k: t[k].cpu().numpy() for k in ("gate_packed", "gate_scales", "up_packed", "up_scales",
                                            "down_packed", "down_scales")}
    x_np, idx_r, w_r, logits, ch = _certified(spec, 0)
    x, idx, w, out, _ = _rf(layer, x_np)
    assert np.array_equal(idx, idx_r)
    used = sorted(set(idx_r.ravel().tolist()))
    es = oracle.ExpertSet(used, spec.n_experts, host["gate_packed"][used], host["gate_scales"][used],
                          host["up_packed"][used], host["up_scales"][used], host["down_packed"][used],
                          host["down_scales"][used])
    ref, denom, _ = oracle.forward(x_np, idx_r, w_r, es, spec.hidden, spec.inter,
                                   shared=synth.make_shared(spec))
    assert rel_err(out, ref, denom) <= REL_TOL


def test_fused_path_falls_back_for_batches_and_latent():
    # T > 1 and a latent layer take route then forward: results as those calls
    spec = synth.LayerSpec(hidden=512, inter=256, n_experts=8, topk=2, shared_inter=256, seed=87,
                           bias_std=0.05, latent=256, latent_norm=1, rms_eps=1e-5)
    t, layer = _make(spec)
    for T in (1, 5):
        x_np = synth.make_x(spec, T)
        x, idx, w, out, _ = _rf(layer, x_np)
        i2, w2, _ = _route(layer, x)
        assert np.array_equal(i2, idx) and np.array_equal(w2, w)
        o2 = torch.empty((T, spec.hidden), dtype=torch.float32, device=DEV)
        layer.forward(x, torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV), o2)
        torch.cuda.synchronize()
        assert np.array_equal(o2.cpu().numpy(), out)
