"""GPU tests of the expert slot cache (k3moe_cache_*): routed experts in
pinned host memory, an HBM arena of slots in front of them.

Bars (integer work bit-exact, the expert arithmetic unchanged):
  - after every call the device slot table and counters equal those of the
    policy model (oracle/cache_policy.py) fed the same assignments;
  - the output is bit-identical to k3moe_forward of the same layer with its
    experts resident in HBM, on the same routes with every assignment the
    model drops replaced by an out-of-range id (which contributes nothing);
  - the output is within the layer's error bound of the fp64 oracle's on
    those routes (every call, every token);
  - dropped assignments are counted by the layer's error counter.
Every input is seeded and synthetic; expected values come only from
``oracle``."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import REL_TOL, oracle_forward, rel_err
from oracle.cache_policy import SlotCache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
_EXPERT_KEYS = ("gate_packed", "gate_scales", "up_packed", "up_scales", "down_packed", "down_scales")


def _pinned(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def _setup(spec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import synth.device as sd
    t = sd.layer_tensors(spec, 0, DEV)
    th = dict(t)
    for k in _EXPERT_KEYS:
        th[k] = _pinned(t[k])
    torch.cuda.synchronize()
    return sd.make_layer(spec, t), sd.make_layer(spec, th), th


def _expert_bytes(spec):
    I, EK = spec.inter, spec.ek
    return 3 * (I * EK // 2 + I * EK // 32)


def _routes(rng, spec, T):
    idx = np.stack([rng.choice(spec.n_experts, spec.topk, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.01, 1.0, (T, spec.topk)).astype(np.float32)
    return idx, w


def _call(spec, cache, model, resident, host, T, rng, attempt):
    import synth.device as sd
    idx, w = _routes(rng, spec, T)
    x_np = synth.make_x(spec, T, attempt=attempt)
    x = sd.bf16_tensor(x_np, DEV)
    idx_d, w_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)
    err0 = host.error_count()
    out_c = torch.empty((T, spec.hidden), dtype=torch.float32, device=DEV)
    print(f"[cache] E={spec.n_experts} S={cache.n_slots} T={T} call {attempt}", flush=True)
    cache.forward(x, idx_d, w_d, out_c)
    slot_map, reads = model.step(idx, _expert_bytes(spec))
    assert cache.slots() == model.key
    assert cache.stats() == model.stats
    dropped = np.array(slot_map).reshape(idx.shape) < 0
    idx_ref = np.where(dropped, -1, idx).astype(np.int32)
    out_r = torch.empty_like(out_c)
    err1 = resident.error_count()
    resident.forward(x, torch.from_numpy(idx_ref).to(DEV), w_d, out_r)
    torch.cuda.synchronize()
    assert np.array_equal(out_c.cpu().numpy(), out_r.cpu().numpy())
    ref, denom, drops = oracle_forward(spec, x_np, idx_ref, w)
    assert drops == int(dropped.sum())
    assert rel_err(out_c.cpu().numpy(), ref, denom) <= REL_TOL
    assert host.error_count() - err0 == int(dropped.sum())
    assert resident.error_count() - err1 == int(dropped.sum())
    return reads, int(dropped.sum())


def _sequence(spec, S, Ts, seed):
    resident, host, _ = _setup(spec)
    import mxfp4_routed_expert_sigmoid_amd as k3
    cache = k3.Cache(host, S)
    model = SlotCache(S, spec.n_experts)
    rng = np.random.default_rng(seed)
    total_drops = total_reads = 0
    for i, T in enumerate(Ts):
        reads, drops = _call(spec, cache, model, resident, host, T, rng, i)
        total_reads += len(reads)
        total_drops += drops
    return cache, model, total_reads, total_drops, resident, host


def test_tiny_cache_sequence_with_evictions_and_drops():
    spec = synth.LayerSpec(hidden=256, inter=128, n_experts=8, topk=2, shared_inter=128,
                           bias_std=0.0, seed=200)
    cache, model, reads, drops, *_ = _sequence(spec, 3, [1, 1, 2, 1, 3, 1, 2, 2, 1, 3, 1, 1], 0)
    assert reads > 3 and drops > 0 and model.stats["evictions"] > 0


def test_mid_cache_stream_and_gemm_paths():
    spec = synth.LayerSpec(hidden=512, inter=256, n_experts=16, topk=4, shared_inter=256,
                           bias_std=0.0, seed=201)
    cache, model, reads, drops, *_ = _sequence(spec, 12, [1, 5, 17, 2, 40, 1], 1)
    assert model.stats["resident_hits"] > 0 and model.stats["evictions"] > 0


def test_latent_layer_through_the_cache():
    spec = synth.LayerSpec(hidden=1024, inter=512, n_experts=16, topk=4, shared_inter=512,
                           bias_std=0.0, seed=202, latent=512)
    _sequence(spec, 8, [1, 3, 1, 9], 2)


def test_full_expert_shape_decode():
    # hidden 7168, inter 1536 experts (17,547,264 B each), 64 of them in host
    # memory, 24 slots, top-16
    spec = synth.LayerSpec(hidden=7168, inter=1536, n_experts=64, topk=16, shared_inter=1536,
                           bias_std=0.0, seed=203)
    cache, model, reads, drops, *_ = _sequence(spec, 24, [1, 1, 1, 1, 2, 1], 3)
    assert drops > 0 and model.stats["bytes_read"] == reads * 17547264


def test_back_to_back_calls_share_the_workspace():
    # Calls of 1..4 tokens issued one after another on one stream with one
    # workspace and no host synchronisation in between: each call's resident
    # experts run on the cache's own stream while its reads are in flight, so
    # the next call's work must wait for this call's combine. Every output must
    # equal the resident layer's on the same (drop-adjusted) routes.
    import synth.device as sd
    import mxfp4_routed_expert_sigmoid_amd as k3
    spec = synth.LayerSpec(hidden=256, inter=128, n_experts=8, topk=2, shared_inter=128,
                           bias_std=0.0, seed=204)
    resident, host, _ = _setup(spec)
    cache = k3.Cache(host, 3)
    model = SlotCache(3, spec.n_experts)
    rng = np.random.default_rng(4)
    Ts = [1, 2, 4, 1, 3, 2, 1, 4, 1, 1]
    ws = cache.workspace(max(Ts))
    calls = []
    for i, T in enumerate(Ts):
        idx, w = _routes(rng, spec, T)
        x_np = synth.make_x(spec, T, attempt=50 + i)
        x = sd.bf16_tensor(x_np, DEV)
        idx_d, w_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)
        out = torch.empty((T, spec.hidden), dtype=torch.float32, device=DEV)
        print(f"[cache] back-to-back call {i} T={T}", flush=True)
        cache.forward(x, idx_d, w_d, out, workspace=ws)
        calls.append((x, idx, w_d, out))
    torch.cuda.synchronize()
    for i, (x, idx, w_d, out) in enumerate(calls):
        slot_map, _ = model.step(idx, _expert_bytes(spec))
        dropped = np.array(slot_map).reshape(idx.shape) < 0
        idx_ref = np.where(dropped, -1, idx).astype(np.int32)
        out_r = torch.empty_like(out)
        resident.forward(x, torch.from_numpy(idx_ref).to(DEV), w_d, out_r)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), out_r.cpu().numpy()), f"call {i}"
    assert cache.slots() == model.key
    assert cache.stats() == model.stats
    assert model.stats["misses"] > 0 and model.stats["resident_hits"] > 0


def test_reset_and_refusals():
    import mxfp4_routed_expert_sigmoid_amd as k3
    spec = synth.LayerSpec(hidden=256, inter=128, n_experts=8, topk=2, shared_inter=0,
                           bias_std=0.0, seed=204)
    resident, host, _ = _setup(spec)
    for bad in (0, -1, 9):
        with pytest.raises(k3.K3MoeError):
            k3.Cache(host, bad)
    cache = k3.Cache(host, 4)
    model = SlotCache(4, 8)
    rng = np.random.default_rng(4)
    _call(spec, cache, model, resident, host, 3, rng, 0)
    cache.reset()
    torch.cuda.synchronize()
    assert cache.slots() == [-1] * 4 and all(v == 0 for v in cache.stats().values())
    model = SlotCache(4, 8)
    _call(spec, cache, model, resident, host, 2, rng, 1)
    # T = 0 does nothing
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    cache.forward(x, torch.empty((0, 2), dtype=torch.int32, device=DEV),
                  torch.empty((0, 2), dtype=torch.float32, device=DEV),
                  torch.empty((0, 256), dtype=torch.float32, device=DEV))
    assert cache.stats() == model.stats
