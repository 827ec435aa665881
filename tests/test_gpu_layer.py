"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every input is seeded and synthetic (``synth``); expected values come only
from ``oracle``."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (REL_TOL, W_RTOL_WAVE, certify_rows, check_logits, check_route, logit_magnitudes,
                         oracle_forward, rel_err, route_certificate, tile_edge_tokens)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import synth.device as sd
    return sd


def _x_dev(x):
    import synth.device as sd
    return sd.bf16_tensor(x, DEV)


def _route_gpu(layer, x_np, T, K, logits=False):
    x = _x_dev(x_np)
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    lg = torch.empty((T, layer.cfg.n_experts), dtype=torch.float32, device=DEV) if logits else None
    layer.route(x, idx, w, logits=lg)
    torch.cuda.synchronize()
    return x, idx, w, lg


def _forward_gpu(layer, x, idx_np, w_np):
    T, K = idx_np.shape
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).to(DEV)
    w = torch.from_numpy(np.ascontiguousarray(w_np, np.float32)).to(DEV)
    out = torch.empty((T, layer.cfg.hidden), dtype=torch.float32, device=DEV)
    layer.forward(x, idx, w, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _certified_x(spec, T, Wr, bias, min_gap=None, max_attempts=50):
    """Token batch whose oracle route is certified on every token (redraws
    the batch with the next attempt number otherwise)."""
    for attempt in range(max_attempts):
        x = synth.make_x(spec, T, attempt=attempt)
        idx, w, logits, ch = oracle.route(x, Wr, bias, spec.topk, want_detail=True)
        ok = route_certificate(ch, spec.topk).all()
        if min_gap is not None:
            s = np.sort(logits, axis=1)
            ok = ok and bool(np.all(np.diff(s, axis=1) >= min_gap))
        if ok:
            return x, idx, w, logits, ch, attempt
    raise AssertionError("no certified batch")


# --------------------------------------------------------------------------
# Tiny layer (hidden 256, 8 experts, top-2, inter 128, no shared expert)

def _tiny(seed=0, **kw):
    spec = synth.tiny_spec(seed=seed)
    for k, v in kw.items():
        setattr(spec, k, v)
    sd = _dev()
    t = sd.layer_tensors(spec, 0, DEV)
    return spec, t, sd.make_layer(spec, t)


def test_tiny_route_and_forward_T1():
    spec, t, layer = _tiny()
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    x_np, idx_r, w_r, logits, ch, _ = _certified_x(spec, 1, Wr, bias, min_gap=1e-3)
    x, idx, w, lg = _route_gpu(layer, x_np, 1, spec.topk, logits=True)
    assert np.array_equal(idx.cpu().numpy(), idx_r)
    assert np.array_equal(w.cpu().numpy(), w_r)
    assert np.array_equal(lg.cpu().numpy(), logits.astype(np.float32))
    out = _forward_gpu(layer, x, idx.cpu().numpy(), w.cpu().numpy())
    ref, denom, drops = oracle_forward(spec, x_np, idx_r, w_r)
    assert drops == 0 and layer.error_count() == 0
    assert rel_err(out, ref, denom) <= REL_TOL


@pytest.mark.parametrize("T", [2, 5, 16, 17, 40, 129])
def test_tiny_ragged_batches(T):
    spec, t, layer = _tiny(seed=1, bias_std=0.05)
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    x_np = synth.make_x(spec, T)
    idx_r, w_r, logits, ch = oracle.route(x_np, Wr, bias, spec.topk, want_detail=True)
    x, idx, w, lg = _route_gpu(layer, x_np, T, spec.topk, logits=True)
    check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk)
    check_logits(lg.cpu().numpy(), logits, ch, bias, logit_magnitudes(x_np, Wr))
    out = _forward_gpu(layer, x, idx_r, w_r)
    ref, denom, _ = oracle_forward(spec, x_np, idx_r, w_r)
    assert rel_err(out, ref, denom) <= REL_TOL


def test_tiny_swiglu_and_no_renorm():
    spec, t, layer = _tiny(seed=2, act=oracle.ACT_SWIGLU, renorm=0, routed_scale=1.5)
    x_np = synth.make_x(spec, 7)
    idx_r, w_r = oracle.route(x_np, synth.make_router(spec), None, spec.topk, renorm=0,
                              routed_scale=1.5)
    out = _forward_gpu(layer, _x_dev(x_np), idx_r, w_r)
    ref, denom, _ = oracle_forward(spec, x_np, idx_r, w_r)
    assert rel_err(out, ref, denom) <= REL_TOL


def test_tiny_scale_edge_bytes():
    # scale byte 255 drops a group; byte 0 is 2^-127 and must not flush
    spec, t, layer = _tiny(seed=3)
    g = torch.Generator().manual_seed(0)
    for name in ("gate_scales", "up_scales", "down_scales"):
        s = t[name]
        m = torch.rand(s.shape, generator=g) < 0.05
        s[m.to(DEV)] = 255
        m0 = torch.rand(s.shape, generator=g) < 0.02
        s[m0.to(DEV)] = 0
    torch.cuda.synchronize()
    x_np = synth.make_x(spec, 3)
    idx_r, w_r = oracle.route(x_np, synth.make_router(spec), None, spec.topk)
    out = _forward_gpu(layer, _x_dev(x_np), idx_r, w_r)
    used = sorted(set(idx_r.ravel().tolist()))
    es = oracle.ExpertSet(used, spec.n_experts, *(t[k][used].cpu().numpy() for k in (
        "gate_packed", "gate_scales", "up_packed", "up_scales", "down_packed", "down_scales")))
    ref, denom, _ = oracle.forward(x_np, idx_r, w_r, es, spec.hidden, spec.inter)
    assert rel_err(out, ref, denom) <= REL_TOL


def test_tiny_invariants_poison_double_relabel():
    spec, t, layer = _tiny(seed=4)
    x_np = synth.make_x(spec, 6)
    idx_r, w_r = oracle.route(x_np, synth.make_router(spec), None, spec.topk)
    x = _x_dev(x_np)
    base = _forward_gpu(layer, x, idx_r, w_r)
    # determinism
    assert np.array_equal(base, _forward_gpu(layer, x, idx_r, w_r))
    # poison every unselected expert: random bytes, scale 254
    used = set(idx_r.ravel().tolist())
    g = torch.Generator().manual_seed(1)
    saved = {k: v.clone() for k, v in t.items() if v is not None and v.dtype == torch.uint8}
    for e in range(spec.n_experts):
        if e in used:
            continue
        for k in saved:
            if k.endswith("packed"):
                t[k][e] = torch.randint(0, 256, t[k][e].shape, generator=g, dtype=torch.uint8).to(DEV)
            else:
                t[k][e] = 254
    assert np.array_equal(base, _forward_gpu(layer, x, idx_r, w_r))
    for k, v in saved.items():
        t[k].copy_(v)
    # +1 on every down scale doubles the (routed-only) output exactly
    t["down_scales"] += 1
    assert np.array_equal(_forward_gpu(layer, x, idx_r, w_r), 2.0 * base)
    t["down_scales"] -= 1
    # relabelling experts (storage, router rows, ids) changes nothing
    perm = np.random.default_rng(2).permutation(spec.n_experts)
    inv = torch.from_numpy(np.argsort(perm)).to(DEV)
    t2 = dict(t)
    for k in saved:
        t2[k] = t[k][inv].contiguous()
    t2["router_w"] = t["router_w"][inv].contiguous()
    import synth.device as sd
    layer2 = sd.make_layer(spec, t2)
    assert np.array_equal(base, _forward_gpu(layer2, x, perm[idx_r], w_r))


@pytest.mark.parametrize("n_experts,groups,bias", [(128, 8, False), (128, 1, False), (128, 1, True),
                                                    (16, 4, False), (896, 7, False)])
def test_route_exact_ties(n_experts, groups, bias):
    # router rows repeat with period `groups`, so experts e and e + groups tie
    # exactly: equal selection scores go to the lowest expert index. With one
    # group and no bias every expert ties (more than 64 candidates in the
    # threshold step: the round-by-round fallback); 8 groups give 16 tied
    # copies of each logit (the rank step with ties)
    spec = synth.LayerSpec(hidden=256, inter=128, n_experts=n_experts, topk=8, shared_inter=0,
                           bias_std=0.05 if bias else 0.0, seed=80 + groups)
    sd = _dev()
    t = sd.layer_tensors(spec, 0, DEV)
    Wr = synth.make_router(spec)[np.arange(n_experts) % groups]
    t["router_w"].copy_(sd.bf16_tensor(np.ascontiguousarray(Wr), DEV))
    layer = sd.make_layer(spec, t)
    bias_np = synth.make_bias(spec)
    x_np = synth.make_x(spec, 5)
    idx_r, w_r = oracle.route(x_np, Wr, bias_np, spec.topk)
    _, idx, w, _ = _route_gpu(layer, x_np, 5, spec.topk)
    assert np.array_equal(idx.cpu().numpy(), idx_r)
    np.testing.assert_allclose(w.cpu().numpy(), w_r, rtol=4e-7, atol=0)


def test_tiny_bad_ids_are_counted():
    spec, t, layer = _tiny(seed=5)
    x_np = synth.make_x(spec, 4)
    idx_r, w_r = oracle.route(x_np, synth.make_router(spec), None, spec.topk)
    x = _x_dev(x_np)
    bad = idx_r.copy()
    bad[0, 1] = -1
    bad[2, 0] = spec.n_experts
    layer.error_reset()
    out_bad = _forward_gpu(layer, x, bad, w_r)
    assert layer.error_count() == 2
    w0 = w_r.copy()
    w0[0, 1] = 0.0
    w0[2, 0] = 0.0
    assert np.array_equal(out_bad, _forward_gpu(layer, x, idx_r, w0))


# --------------------------------------------------------------------------
# Mid-size layer (hidden 512, inter 512, 16 experts, top-4, shared 256): the
# sizes that take the weight-streaming kernels for experts with at most 16
# tokens and the grouped GEMMs for the rest; the shared expert streams for
# batches up to 128 tokens and runs as a GEMM above that.

def _mid(seed, routing="normal", T_bad=False):
    spec = synth.LayerSpec(hidden=512, inter=512, n_experts=16, topk=4, shared_inter=256,
                           bias_std=0.05, routing=routing, seed=seed)
    sd = _dev()
    t = sd.layer_tensors(spec, 0, DEV)
    return spec, t, sd.make_layer(spec, t)


@pytest.mark.parametrize("T,routing", [(1, "normal"), (2, "normal"), (5, "normal"), (9, "normal"), (17, "normal"),
                                       (40, "normal"), (128, "normal"), (129, "zipf"), (300, "zipf")])
def test_mid_stream_and_gemm_mix(T, routing):
    spec, t, layer = _mid(seed=20 + T, routing=routing)
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    x_np = synth.make_x(spec, T)
    idx_r, w_r, logits, ch = oracle.route(x_np, Wr, bias, spec.topk, want_detail=True)
    x, idx, w, _ = _route_gpu(layer, x_np, T, spec.topk)
    check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk)
    counts = np.bincount(idx_r.ravel(), minlength=spec.n_experts)
    if T >= 129:
        assert counts.max() > 16 and 0 < counts[counts > 0].min() <= 16  # both kernel kinds run
    out = _forward_gpu(layer, x, idx_r, w_r)
    ref, denom, _ = oracle_forward(spec, x_np, idx_r, w_r)
    assert rel_err(out, ref, denom) <= REL_TOL
    # deterministic: a second call gives the same bits
    assert np.array_equal(out, _forward_gpu(layer, x, idx_r, w_r))


def test_mid_bad_ids_are_counted():
    spec, t, layer = _mid(seed=40)
    T = 24
    x_np = synth.make_x(spec, T)
    idx_r, w_r = oracle.route(x_np, synth.make_router(spec), synth.make_bias(spec), spec.topk)
    x = _x_dev(x_np)
    bad = idx_r.copy()
    bad[0, 1] = -1
    bad[5, 0] = spec.n_experts
    bad[23, 3] = 1 << 30
    layer.error_reset()
    out_bad = _forward_gpu(layer, x, bad, w_r)
    assert layer.error_count() == 3
    ref, denom, drops = oracle_forward(spec, x_np, bad, w_r)
    assert drops == 3
    assert rel_err(out_bad, ref, denom) <= REL_TOL


def test_empty_batch_is_a_no_op():
    spec, t, layer = _tiny(seed=6)
    x = torch.empty((0, spec.hidden), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((0, spec.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((0, spec.topk), dtype=torch.float32, device=DEV)
    out = torch.empty((0, spec.hidden), dtype=torch.float32, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    layer.route(x, idx, w, workspace=ws)
    layer.forward(x, idx, w, out, workspace=ws)


@pytest.mark.parametrize("T,shared", [(1, 0), (3, 0), (3, 3072), (40, 3072)])
def test_pages_expert_shape(T, shared):
    # the README's latent expert shape (width 3584, intermediate 3072), few
    # experts: one token, light experts, and heavy ones (40 tokens x top-3
    # over 6 experts), with and without a shared expert of that width
    spec = synth.LayerSpec(hidden=3584, inter=3072, n_experts=6, topk=3, shared_inter=shared,
                           bias_std=0.01, seed=8)
    sd = _dev()
    layer = sd.make_layer(spec, sd.layer_tensors(spec, 0, DEV))
    x_np = synth.make_x(spec, T)
    idx_r, w_r = oracle.route(x_np, synth.make_router(spec), synth.make_bias(spec), spec.topk)
    out = _forward_gpu(layer, _x_dev(x_np), idx_r, w_r)
    ref, denom, _ = oracle_forward(spec, x_np, idx_r, w_r)
    assert rel_err(out, ref, denom) <= REL_TOL


@pytest.mark.parametrize("T,inter,hidden", [(1, 3200, 256), (1, 2176, 256), (1, 1664, 256), (2, 3200, 256),
                                           (1, 3584, 512)])
def test_inter_widths_past_and_below_decode_staging(T, inter, hidden):
    # intermediate widths that are not multiples of 512, one past the
    # single-token down kernel's activation staging (3072 elements: such a
    # layer takes the grouped path) and two within it; and 3584 at hidden
    # 512, where one token takes the streaming kernels with the shared
    # expert cut into hidden-dimension slices (their partials need room in
    # the workspace at T = 1 too)
    spec = synth.LayerSpec(hidden=hidden, inter=inter, n_experts=4, topk=2, shared_inter=128,
                           bias_std=0.05, seed=70 + inter)
    sd = _dev()
    layer = sd.make_layer(spec, sd.layer_tensors(spec, 0, DEV))
    x_np = synth.make_x(spec, T)
    idx_r, w_r = oracle.route(x_np, synth.make_router(spec), synth.make_bias(spec), spec.topk)
    out = _forward_gpu(layer, _x_dev(x_np), idx_r, w_r)
    ref, denom, _ = oracle_forward(spec, x_np, idx_r, w_r)
    assert rel_err(out, ref, denom) <= REL_TOL


@pytest.mark.parametrize("T,routing", [(1, "normal"), (5, "normal"), (129, "zipf")])
def test_mid_swiglu_no_renorm(T, routing):
    # SwiGLU, no renormalisation, a routed scale: the single-token kernels,
    # the streaming kernels and the grouped GEMMs
    spec = synth.LayerSpec(hidden=512, inter=512, n_experts=16, topk=4, shared_inter=256,
                           bias_std=0.05, routing=routing, seed=60 + T, act=oracle.ACT_SWIGLU,
                           renorm=0, routed_scale=2.5)
    sd = _dev()
    layer = sd.make_layer(spec, sd.layer_tensors(spec, 0, DEV))
    x_np = synth.make_x(spec, T)
    idx_r, w_r, _, ch = oracle.route(x_np, synth.make_router(spec), synth.make_bias(spec), spec.topk,
                                     renorm=0, routed_scale=2.5, want_detail=True)
    x, idx, w, _ = _route_gpu(layer, x_np, T, spec.topk)
    check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk)
    out = _forward_gpu(layer, x, idx_r, w_r)
    ref, denom, _ = oracle_forward(spec, x_np, idx_r, w_r)
    assert rel_err(out, ref, denom) <= REL_TOL


# --------------------------------------------------------------------------
# Full shape (hidden 7168, 896 experts, top-16, inter 1536, bf16 shared expert)

_FULL = {}


def _full(routing="normal"):
    if routing not in _FULL:
        sd = _dev()
        spec = synth.full_spec(seed=0, routing=routing)
        t = sd.layer_tensors(spec, 0, DEV)
        _FULL.clear()
        _FULL[routing] = (spec, t, sd.make_layer(spec, t))
    return _FULL[routing]


def test_full_device_bytes_match_host_generator():
    spec, t, _ = _full()
    k = synth.stream_key(spec.seed, 0, synth.DOWN_PACKED)
    e = 777
    n = spec.hidden * spec.inter // 2
    host = synth.packed_bytes(k, e * n + 4096, 4096)
    assert np.array_equal(t["down_packed"][e].reshape(-1)[4096:8192].cpu().numpy(), host)
    ks = synth.stream_key(spec.seed, 0, synth.UP_SCALES)
    ns = spec.hidden * spec.inter // 32
    assert np.array_equal(t["up_scales"][e].reshape(-1)[:1000].cpu().numpy(),
                          synth.scale_bytes(ks, e * ns, 1000))


def test_full_decode_T1():
    spec, t, layer = _full()
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    x_np, idx_r, w_r, logits, ch, _ = _certified_x(spec, 1, Wr, bias)
    x, idx, w, lg = _route_gpu(layer, x_np, 1, spec.topk, logits=True)
    assert check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk, w_rtol=W_RTOL_WAVE) == 1
    l32 = logits.astype(np.float32)
    assert np.max(np.abs(lg.cpu().numpy() - l32) / np.maximum(np.abs(l32), 1e-30)) <= 2.0 ** -23
    out = _forward_gpu(layer, x, idx_r, w_r)
    ref, denom, _ = oracle_forward(spec, x_np, idx_r, w_r)
    assert rel_err(out, ref, denom) <= REL_TOL
    # bitwise reproducible
    assert np.array_equal(out, _forward_gpu(layer, x, idx_r, w_r))


@pytest.mark.parametrize("T", [3, 4, 8])
def test_full_small_batch_per_token(T):
    # batches of up to 8 tokens run the single-token kernels once per token,
    # sharing one token's workspace rows in stream order
    spec, t, layer = _full()
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    x_np, idx_r, w_r, logits, ch, _ = _certified_x(spec, T, Wr, bias)
    x, idx, w, _ = _route_gpu(layer, x_np, T, spec.topk)
    assert check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk, w_rtol=W_RTOL_WAVE) == T
    out = _forward_gpu(layer, x, idx_r, w_r)
    ref, denom, _ = oracle_forward(spec, x_np, idx_r, w_r)
    assert rel_err(out, ref, denom) <= REL_TOL
    assert np.array_equal(out, _forward_gpu(layer, x, idx_r, w_r))


def test_full_batched_decode_T64_all_tokens():
    # every token of the batch certified (uncertified ones redrawn), so the
    # GPU's ids equal the oracle's on all 64; every output compared
    spec, t, layer = _full()
    T = 64
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    x_np = synth.make_x(spec, T, attempt=1)
    idx_r, w_r, logits, ch = certify_rows(spec, x_np, Wr, bias)
    x, idx, w, lg = _route_gpu(layer, x_np, T, spec.topk, logits=True)
    assert check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk) == T
    dl, dch = check_logits(lg.cpu().numpy(), logits, ch, bias, logit_magnitudes(x_np, Wr))
    out = _forward_gpu(layer, x, idx_r, w_r)
    ref, denom, drops = oracle_forward(spec, x_np, idx_r, w_r)
    assert drops == 0
    err = rel_err(out, ref, denom)
    print(f"[full T=64] max rel err {err:.3g} over {T} tokens; logits: {dl:.3g} of the magnitude sum beyond "
          f"one ulp, selection scores within {dch:.3g}", flush=True)
    assert err <= REL_TOL
    assert layer.error_count() == 0


# Tile geometry of the multi-token path at this shape (a flat layer, one bf16
# plane): experts with more than 16 assignments run on 128-token gate/up tiles
# and 64-token down tiles; the others stream.
_SMAX, _TILE_GU, _TILE_DN = 16, 128, 64


def test_full_prefill_T2048_zipf_tile_edges():
    # 2048 Zipf-routed tokens, all certified (so the GPU's ids equal the
    # oracle's on every token and the tiles are the ones the oracle's ids
    # give); compared: every token on a tile edge of every expert that runs on
    # tiles (first/last row of its first and last gate/up and down tile, the
    # first row of its second), plus 32 drawn at random
    spec, t, layer = _full("zipf")
    T = 2048
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    x_np = synth.make_x(spec, T)
    idx_r, w_r, logits, ch = certify_rows(spec, x_np, Wr, bias)
    x, idx, w, lg = _route_gpu(layer, x_np, T, spec.topk, logits=True)
    assert check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk) == T
    dl, dch = check_logits(lg.cpu().numpy(), logits, ch, bias, logit_magnitudes(x_np, Wr))
    print(f"[full T=2048 zipf] logits: {dl:.3g} of the magnitude sum beyond one ulp, selection scores "
          f"within {dch:.3g}", flush=True)
    out = _forward_gpu(layer, x, idx_r, w_r)
    assert layer.error_count() == 0
    edges = tile_edge_tokens(idx_r, spec.n_experts, _SMAX, (_TILE_GU, _TILE_DN))
    counts = np.bincount(idx_r.ravel(), minlength=spec.n_experts)
    assert (counts > _SMAX).sum() >= 32 and counts.max() > 8 * _TILE_GU   # the tile path is exercised
    rng = np.random.default_rng(0)
    check = np.union1d(edges, rng.choice(T, 32, replace=False))
    assert check.size >= 64
    ref, denom, drops = oracle_forward(spec, x_np, idx_r, w_r, tokens=check)
    assert drops == 0
    err = rel_err(out[check], ref, denom)
    print(f"[full T=2048 zipf] max rel err {err:.3g} over {check.size} tokens "
          f"({len(edges)} on tile edges of {(counts > _SMAX).sum()} experts)", flush=True)
    assert err <= REL_TOL


@pytest.mark.parametrize("latent", [0, 256])
def test_repeated_ids_within_a_token(latent):
    # a token may name an expert more than once (the layer sums every
    # assignment): an expert's item then holds more assignments than there
    # are tokens, which the streaming kernels stage once per distinct token
    spec = synth.LayerSpec(hidden=512, inter=512, n_experts=16, topk=4, shared_inter=256,
                           bias_std=0.05, seed=77, latent=latent)
    sd = _dev()
    t = sd.layer_tensors(spec, 0, DEV)
    layer = sd.make_layer(spec, t)
    rng = np.random.default_rng(7)
    cases = [np.array([[5, 5, 5, 5]]),
             np.array([[5, 5, 5, 2], [5, 7, 7, 1], [5, 3, 9, 9]]),
             np.array([[1, 1, 4, 4], [4, 4, 1, 1]])]
    for idx in cases:
        T = idx.shape[0]
        idx = idx.astype(np.int32)
        w = rng.uniform(0.05, 1.0, idx.shape).astype(np.float32)
        x_np = synth.make_x(spec, T, attempt=T)
        out = _forward_gpu(layer, _x_dev(x_np), idx, w)
        ref, denom, drops = oracle_forward(spec, x_np, idx, w)
        assert drops == 0
        assert rel_err(out, ref, denom) <= REL_TOL, idx.tolist()


@pytest.mark.parametrize("n_experts,topk", [(8, 8), (8, 1), (1, 1), (4, 4)])
def test_degenerate_routing(n_experts, topk):
    # every expert selected (top-k = E), a single expert per token, a single
    # expert in the layer: routes and outputs against the oracle
    spec = synth.LayerSpec(hidden=256, inter=128, n_experts=n_experts, topk=topk, shared_inter=128,
                           bias_std=0.05, seed=300 + 10 * n_experts + topk)
    sd = _dev()
    t = sd.layer_tensors(spec, 0, DEV)
    layer = sd.make_layer(spec, t)
    for T in (1, 7):
        Wr, bias = synth.make_router(spec), synth.make_bias(spec)
        x_np = synth.make_x(spec, T)
        idx_r, w_r, _, ch = oracle.route(x_np, Wr, bias, spec.topk, want_detail=True)
        x, idx, w, _ = _route_gpu(layer, x_np, T, spec.topk)
        check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk)
        if topk == n_experts:  # every expert, in descending selection score
            assert all(sorted(r) == list(range(n_experts)) for r in idx.cpu().numpy().tolist())
        out = _forward_gpu(layer, x, idx_r, w_r)
        ref, denom, _ = oracle_forward(spec, x_np, idx_r, w_r)
        assert rel_err(out, ref, denom) <= REL_TOL


def test_full_largest_batch_and_one_past_it():
    # the largest batch the 32-bit batch offsets take at this shape
    # (T * topk * inter * 2 bytes below 2 GiB: T = 43,690), sampled tokens
    # against the oracle; one token more is refused before any launch
    import mxfp4_routed_expert_sigmoid_amd as k3
    spec, t, layer = _full()
    T = 43690
    x_np = synth.make_x(spec, T, attempt=3)
    sample = [0, 12345, 30001, T - 1]
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    idx_r, w_r, _, ch = certify_rows(spec, x_np, Wr, bias, rows=sample)
    x, idx, w, _ = _route_gpu(layer, x_np, T, spec.topk)
    idx_g, w_g = idx.cpu().numpy(), w.cpu().numpy()
    assert check_route(idx_g[sample], w_g[sample], idx_r, w_r, ch, spec.topk) == len(sample)
    out = _forward_gpu(layer, x, idx_g, w_g)
    # plus the tile edges of the two most loaded experts (ids as run: the GPU's)
    counts = np.bincount(idx_g.ravel(), minlength=spec.n_experts)
    hot = np.argsort(-counts, kind="stable")[:2]
    check = np.union1d(sample, tile_edge_tokens(idx_g, spec.n_experts, _SMAX, (_TILE_GU, _TILE_DN), hot))
    ref, denom, _ = oracle_forward(spec, x_np, idx_g, w_g, tokens=check)
    assert rel_err(out[check], ref, denom) <= REL_TOL
    del out
    with pytest.raises(k3.K3MoeError):
        layer.workspace_size(T + 1)
    big = torch.empty((T + 1, spec.hidden), dtype=torch.bfloat16, device=DEV)
    i1 = torch.empty((T + 1, spec.topk), dtype=torch.int32, device=DEV)
    w1 = torch.empty((T + 1, spec.topk), dtype=torch.float32, device=DEV)
    ws = layer.workspace(T)
    with pytest.raises(k3.K3MoeError):
        layer.route(big, i1, w1, workspace=ws)
    torch.cuda.synchronize()
