"""The C-ABI library loads, exports what include/k3moe.h declares, and
refuses invalid configs on the host (no GPU needed: validation runs before
any device call)."""
import ctypes
import os
import re

import pytest

import mxfp4_routed_expert_sigmoid_amd as k3
from conftest import ROOT


def _declared():
    src = open(os.path.join(ROOT, "include", "k3moe.h")).read()
    return sorted(set(re.findall(r"\b(k3moe_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(k3.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = k3.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings():
    L = k3.lib()
    for s, text in k3.STATUS.items():
        assert L.k3moe_status_string(s).decode() == text


def _weights(E, shared=False, misalign=False):
    base = 0x10000000 + (8 if misalign else 0)
    mx = k3.MXFP4(base, base + 0x1000000, 0x10000, 0x1000)
    sh = (base + 0x100, base + 0x200, base + 0x300) if shared else (None, None, None)
    return k3.Weights(base, None, mx, mx, mx, *sh)


def _create(cfg, w):
    h = ctypes.c_void_p()
    return k3.lib().k3moe_layer_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h))


@pytest.mark.parametrize("field,value,status", [
    ("struct_size", 4, 2), ("abi_version", 99, 2), ("hidden", 0, 2), ("topk", 9, 2),
    ("act", 0, 2), ("renorm", 2, 2), ("situ_b1", 0.0, 2), ("routed_scale", float("nan"), 2),
    ("hidden", 96, 3), ("inter", 200, 3), ("shared_inter", 64, 3), ("n_experts", 5000, 3),
])
def test_config_refusals(field, value, status):
    cfg = k3.make_config(256, 128, 8, 2)
    setattr(cfg, field, value)
    assert _create(cfg, _weights(8)) == status


def test_weight_descriptor_refusals():
    cfg = k3.make_config(256, 128, 8, 2)
    w = _weights(8)
    w.gate.expert_stride_packed = 100          # smaller than one matrix
    assert _create(cfg, w) == 1
    w = _weights(8)
    w.router_w = None
    assert _create(cfg, w) == 1
    assert _create(cfg, _weights(8, misalign=True)) == 4
    w = _weights(8)
    w.down.scales += 4                           # scales must be 16-byte aligned too
    assert _create(cfg, w) == 4
    w = _weights(8)
    w.up.expert_stride_scales = 0x1008
    assert _create(cfg, w) == 4
    assert _create(cfg, _weights(8, shared=True)) == 1   # shared pointers without shared_inter
    cfg2 = k3.make_config(256, 128, 8, 2, shared_inter=128)
    assert _create(cfg2, _weights(8)) == 1               # shared_inter without pointers


@pytest.mark.parametrize("latent,norm,eps,status", [
    (0, 1, 1e-5, 2),        # a flat layer has no latent norm
    (-128, 0, 0.0, 2),
    (128, 2, 1e-5, 2),      # norm flag 0 or 1
    (128, 1, 0.0, 2),       # the norm needs a positive epsilon
    (128, 1, float("inf"), 2),
    (96, 0, 0.0, 3),        # latent a multiple of 128
])
def test_latent_config_refusals(latent, norm, eps, status):
    cfg = k3.make_config(256, 128, 8, 2, latent=latent, latent_norm=norm, rms_eps=eps)
    assert _create(cfg, _weights(8)) == status


def test_latent_weight_refusals():
    base = 0x20000000
    lat = k3.make_config(256, 128, 8, 2, latent=128, latent_norm=1, rms_eps=1e-5)
    w = _weights(8)                                   # latent layer without its projections
    assert _create(lat, w) == 1
    w.lat_down, w.lat_up = base, base + 0x100000      # norm on, no gamma
    assert _create(lat, w) == 1
    w.lat_norm = base + 0x200004                      # gamma not 16-byte aligned
    assert _create(lat, w) == 4
    flat = k3.make_config(256, 128, 8, 2)
    w2 = _weights(8)
    w2.lat_up = base                                  # projections on a flat layer
    assert _create(flat, w2) == 1
    nonorm = k3.make_config(256, 128, 8, 2, latent=128, latent_norm=0)
    w3 = _weights(8)
    w3.lat_down, w3.lat_up, w3.lat_norm = base, base + 0x100000, base + 0x200000
    assert _create(nonorm, w3) == 1                   # gamma without the norm


def test_stage_list_matches_header():
    src = open(os.path.join(ROOT, "include", "k3moe.h")).read()
    n = int(re.search(r"K3MOE_N_STAGES\s*=\s*(\d+)", src).group(1))
    names = re.findall(r"K3MOE_STAGE_([A-Z_]+)\s*=\s*(\d+)", src)
    assert len(k3.STAGES) == n == len(names)
    for name, i in names:
        assert k3.STAGES[int(i)] == name.lower()
    abi = int(re.search(r"#define K3MOE_ABI_VERSION (\d+)u", src).group(1))
    assert k3.ABI_VERSION == abi


# ---------------------------------------------------------------------------
# The binding refuses mis-shaped tensors before any library call (the C ABI
# takes raw pointers, so a wrong shape would become an out-of-bounds device
# access). These run on the CPU: the shape checks come before the device
# checks, and nothing reaches the library.

def _fake_layer(hidden=256, inter=128, n_experts=8, topk=2):
    import torch
    L = k3.Layer.__new__(k3.Layer)
    L.cfg = k3.make_config(hidden, inter, n_experts, topk)
    L.device = torch.device("cpu")
    L.handle = None
    return L


@pytest.mark.parametrize("call", ["route", "forward", "route_forward", "forward_noalloc",
                                  "forward_residual", "step"])
def test_binding_refuses_mis_shaped_tensors(call):
    import torch
    L = _fake_layer()
    T, H, K, E = 3, 256, 2, 8
    good = dict(x=torch.zeros(T, H, dtype=torch.int16), idx=torch.zeros(T, K, dtype=torch.int32),
                w=torch.zeros(T, K), out=torch.zeros(T, H), h=torch.zeros(T, H),
                gamma=torch.zeros(H), logits=torch.zeros(T, E))
    bad = {"x": torch.zeros(T, H + 128, dtype=torch.int16), "idx": torch.zeros(T, K + 1, dtype=torch.int32),
           "w": torch.zeros(T + 1, K), "out": torch.zeros(T, H - 128), "h": torch.zeros(T, 2 * H),
           "gamma": torch.zeros(H + 1), "logits": torch.zeros(T, E + 1)}
    args = {"route": ("x", "idx", "w"), "forward": ("x", "idx", "w", "out"),
            "route_forward": ("x", "idx", "w", "out"), "forward_noalloc": ("x", "idx", "w", "out"),
            "forward_residual": ("x", "idx", "w", "h"), "step": ("h", "gamma", None, "idx", "w")}[call]
    for wrong in [a for a in args if a]:
        vals = []
        for a in args:
            if a is None:
                vals.append(1e-5)  # step's eps
            else:
                vals.append(bad[a] if a == wrong else good[a])
        with pytest.raises(ValueError, match="shape"):
            getattr(L, call)(*vals)
    if call in ("route", "route_forward"):
        vals = [good[a] for a in args]
        with pytest.raises(ValueError, match="logits"):
            getattr(L, call)(*vals, logits=bad["logits"])


def test_cache_device_bytes_plan_on_the_host():
    # the cache's device allocations from the config alone (no device call):
    # the arena is n_slots slots of the expert's six tensors, each padded to
    # 256 bytes; the slot table adds a little per expert and per slot
    import mxfp4_routed_expert_sigmoid_amd as k3
    cfg = k3.make_config(7168, 1536, 896, 16, 1536)
    slot = 3 * (1536 * 7168 // 2 + 1536 * 7168 // 32)
    assert slot == 17547264
    for S in (1, 24, 224, 896):
        n = k3.cache_device_bytes(cfg, S)
        assert S * slot < n <= S * slot + 256 + 4 * 896 + 12 * S + 3 * 256
    # padding: hidden 384, inter 128 -> packed 24,576 B (aligned), scales 1,536 B (aligned);
    # latent 256, inter 384 -> scales 3,072 B; inter 128, hidden 128 -> scales 512 B
    cfg2 = k3.make_config(128, 128, 4, 2, 0)
    one = k3.cache_device_bytes(cfg2, 1)
    two = k3.cache_device_bytes(cfg2, 2)
    per = 3 * (8192 + 512)
    assert per <= two - one <= per + 3 * 256
    for bad in (0, -1, 5):
        with pytest.raises(k3.K3MoeError) as ei:
            k3.cache_device_bytes(cfg2, bad)
        assert ei.value.status == 1
    with pytest.raises(k3.K3MoeError) as ei:
        k3.cache_device_bytes(k3.make_config(100, 128, 4, 2, 0), 1)   # hidden not a multiple of 128
    assert ei.value.status == 3
