"""Refusals at the C ABI that need a device: a workspace one byte too small,
misaligned or missing gives K3MOE_E_WORKSPACE from every call that takes
one, with nothing launched (outputs, the residual stream and the workspace
keep their bytes; the profiler records no launch); the free-memory budget
(K3MOE_HBM_BUDGET) makes the create calls refuse with
K3MOE_E_OUT_OF_MEMORY before allocating anything.

Calls go through ctypes with explicit pointers and byte counts (the Python
binding would align and size the workspace itself)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
E_WORKSPACE = 5
E_OOM = 6
E_INVALID_ARG = 1


def _layer(spec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import synth.device as sd
    t = sd.layer_tensors(spec, 0, DEV)
    return t, sd.make_layer(spec, t)


def _spec():
    return synth.LayerSpec(hidden=256, inter=128, n_experts=8, topk=2, shared_inter=128,
                           bias_std=0.05, seed=410)


class _Buffers:
    """Sentinel-filled outputs and workspace of one call shape."""

    def __init__(self, spec, T, ws_need):
        H, K, E = spec.hidden, spec.topk, spec.n_experts
        import synth.device as sd
        self.x = sd.bf16_tensor(synth.make_x(spec, T), DEV)
        self.idx = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
        self.w = torch.full((T, K), 0.25, dtype=torch.float32, device=DEV)
        self.logits = torch.full((T, E), -3.0, dtype=torch.float32, device=DEV)
        self.out = torch.full((T, H), 7.0, dtype=torch.float32, device=DEV)
        self.h = torch.full((T, H), 1.5, dtype=torch.float32, device=DEV)
        self.hb = torch.full((T, H), 0x1234, dtype=torch.int16, device=DEV)
        self.gamma = torch.ones(H, dtype=torch.float32, device=DEV)
        self.ws = torch.full((ws_need + 1024,), 0xA5, dtype=torch.uint8, device=DEV)
        base = self.ws.data_ptr()
        self.ws_ptr = base + (-base) % 256          # 256-aligned
        self.need = ws_need

    def snapshot(self):
        torch.cuda.synchronize()
        return [t.clone() for t in (self.idx, self.w, self.logits, self.out, self.h, self.hb, self.ws)]

    def unchanged(self, snap):
        torch.cuda.synchronize()
        now = (self.idx, self.w, self.logits, self.out, self.h, self.hb, self.ws)
        return all(torch.equal(a, b) for a, b in zip(snap, now))


def _bad_workspaces(b):
    """(pointer, bytes) pairs every call must refuse."""
    return [(b.ws_ptr, b.need - 1),            # one byte too small
            (b.ws_ptr + 16, b.need),           # 16-byte but not 256-byte aligned
            (b.ws_ptr + 1, b.need),            # misaligned
            (None, b.need)]                    # missing


def _calls(layer, b, T):
    import mxfp4_routed_expert_sigmoid_amd as k3
    L, hd = k3.lib(), layer.handle
    P = ctypes.c_void_p
    return {
        "route": lambda p, n: L.k3moe_route(hd, b.x.data_ptr(), T, b.idx.data_ptr(), b.w.data_ptr(),
                                            b.logits.data_ptr(), P(p), n, None),
        "forward": lambda p, n: L.k3moe_forward(hd, b.x.data_ptr(), T, b.idx.data_ptr(), b.w.data_ptr(),
                                                b.out.data_ptr(), P(p), n, None),
        "route_forward": lambda p, n: L.k3moe_route_forward(hd, b.x.data_ptr(), T, b.idx.data_ptr(),
                                                            b.w.data_ptr(), b.out.data_ptr(),
                                                            b.logits.data_ptr(), P(p), n, None),
        "forward_residual": lambda p, n: L.k3moe_forward_residual(hd, b.x.data_ptr(), T, b.idx.data_ptr(),
                                                                  b.w.data_ptr(), b.h.data_ptr(),
                                                                  b.hb.data_ptr(), P(p), n, None),
        "step": lambda p, n: L.k3moe_step(hd, b.h.data_ptr(), T, b.gamma.data_ptr(), ctypes.c_float(1e-5),
                                          None, b.idx.data_ptr(), b.w.data_ptr(), b.hb.data_ptr(),
                                          P(p), n, None),
    }


@pytest.mark.parametrize("T", [1, 3])
def test_workspace_refusals_launch_nothing(T):
    spec = _spec()
    _, layer = _layer(spec)
    b = _Buffers(spec, T, layer.workspace_size(T))
    # valid ids for the forward calls
    b.idx.copy_(torch.tensor([[0, 5], [3, 1], [7, 2]][:T], dtype=torch.int32))
    layer.profile(True)
    layer.profile_read()
    for name, call in _calls(layer, b, T).items():
        snap = b.snapshot()
        for p, n in _bad_workspaces(b):
            assert call(p, n) == E_WORKSPACE, (name, p, n)
        assert b.unchanged(snap), name
        launches = sum(c for _, c in layer.profile_read().values())
        assert launches == 0, (name, launches)
    # the exact size at an aligned address is accepted, and launches
    for name, call in _calls(layer, b, T).items():
        b.idx.copy_(torch.tensor([[0, 5], [3, 1], [7, 2]][:T], dtype=torch.int32))
        assert call(b.ws_ptr, b.need) == 0, name
        torch.cuda.synchronize()
        assert sum(c for _, c in layer.profile_read().values()) > 0, name
    layer.profile(False)


def test_cache_workspace_refusals_launch_nothing():
    import mxfp4_routed_expert_sigmoid_amd as k3
    spec = _spec()
    t, layer = _layer(spec)
    cache = k3.Cache(layer, 4)
    T = 3
    b = _Buffers(spec, T, cache.workspace_size(T))
    b.idx.copy_(torch.tensor([[0, 5], [3, 1], [7, 2]], dtype=torch.int32))
    L = k3.lib()
    call = lambda p, n: L.k3moe_cache_forward(cache.handle, b.x.data_ptr(), T, b.idx.data_ptr(),
                                              b.w.data_ptr(), b.out.data_ptr(), ctypes.c_void_p(p), n, None)
    snap = b.snapshot()
    for p, n in _bad_workspaces(b):
        assert call(p, n) == E_WORKSPACE, (p, n)
    assert b.unchanged(snap)
    # no plan ran: the slot table is still empty and the counters zero
    assert cache.slots() == [-1] * 4 and all(v == 0 for v in cache.stats().values())
    assert call(b.ws_ptr, b.need) == 0
    torch.cuda.synchronize()
    assert cache.stats()["steps"] == 1
    cache.close()


class _Budget:
    def __init__(self, value):
        self.value = value

    def __enter__(self):
        os.environ["K3MOE_HBM_BUDGET"] = str(self.value)

    def __exit__(self, *a):
        os.environ.pop("K3MOE_HBM_BUDGET", None)


def test_hbm_budget_refuses_cache_and_layer_before_allocating():
    import mxfp4_routed_expert_sigmoid_amd as k3
    import synth.device as sd
    spec = _spec()
    t, layer = _layer(spec)
    S = 6
    need = k3.cache_device_bytes(layer.cfg, S) + (1 << 20)   # arena + table + the margin
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(DEV)[0]
    with _Budget(need - 1):
        with pytest.raises(k3.K3MoeError) as ei:
            k3.Cache(layer, S)
    assert ei.value.status == E_OOM
    # a layer needs its 8-byte counter and the 1 MiB margin
    with _Budget((1 << 20) + 7):
        with pytest.raises(k3.K3MoeError) as ei:
            sd.make_layer(spec, t)
    assert ei.value.status == E_OOM
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info(DEV)[0] >= free0 - (2 << 20)   # nothing was kept
    for bad in ("12ab", "-5", " 7", "1e9"):
        with _Budget(bad):
            with pytest.raises(k3.K3MoeError) as ei:
                k3.Cache(layer, S)
        assert ei.value.status == E_INVALID_ARG, bad
    with _Budget(need):
        c = k3.Cache(layer, S)   # exactly enough
    assert c.slots() == [-1] * S
    c.close()
    with _Budget((1 << 20) + 8):
        l2 = sd.make_layer(spec, t)
    l2.close()
