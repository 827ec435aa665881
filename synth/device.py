"""Device copies of the seeded synthetic inputs (torch tensors in HBM).

MXFP4 bytes are generated in place by libk3synth.so (the same splitmix64
streams as the host generator); float inputs are drawn on the host by
``synth`` and copied. No layer arithmetic happens here.
"""
import ctypes
import os

import numpy as np
import torch

import synth
from synth import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise ImportError(f"{_build.LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_build.LIB)
        P, i64 = ctypes.c_void_p, ctypes.c_int64
        L.k3synth_fill_packed.restype = ctypes.c_int
        L.k3synth_fill_packed.argtypes = [P, i64, ctypes.c_uint64, i64, P]
        L.k3synth_fill_scales.restype = ctypes.c_int
        L.k3synth_fill_scales.argtypes = [P, i64, ctypes.c_uint64, i64, ctypes.c_int, ctypes.c_int, P]
        L.k3synth_read_probe.restype = ctypes.c_int
        L.k3synth_read_probe.argtypes = [P, i64, P, P]
        _lib = L
    return _lib


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fill_packed(t, key, start=0):
    rc = lib().k3synth_fill_packed(t.data_ptr(), t.numel(), key, start, _stream(t.device))
    if rc != 0:
        raise RuntimeError(f"k3synth_fill_packed failed ({rc})")


def fill_scales(t, key, start=0):
    rc = lib().k3synth_fill_scales(t.data_ptr(), t.numel(), key, start, synth.SCALE_LO,
                                   synth.SCALE_SPAN, _stream(t.device))
    if rc != 0:
        raise RuntimeError(f"k3synth_fill_scales failed ({rc})")


def read_probe(t, sink):
    """Launch the calibration read kernel over tensor t (every byte once)."""
    rc = lib().k3synth_read_probe(t.data_ptr(), t.numel() * t.element_size(), sink.data_ptr(),
                                  _stream(t.device))
    if rc != 0:
        raise RuntimeError(f"k3synth_read_probe failed ({rc})")


def bf16_tensor(bits, device):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def layer_tensors(spec: synth.LayerSpec, layer: int = 0, device="cuda"):
    """All weights of one synthetic layer, resident in HBM."""
    E, H, I = spec.n_experts, spec.ek, spec.inter
    d = {}
    d["router_w"] = bf16_tensor(synth.make_router(spec, layer), device)
    b = synth.make_bias(spec, layer)
    d["router_bias"] = None if b is None else torch.from_numpy(b).to(device)
    for name, tp, ts, rows, cols in (("gate", synth.GATE_PACKED, synth.GATE_SCALES, I, H),
                                     ("up", synth.UP_PACKED, synth.UP_SCALES, I, H),
                                     ("down", synth.DOWN_PACKED, synth.DOWN_SCALES, H, I)):
        p = torch.empty((E, rows, cols // 2), dtype=torch.uint8, device=device)
        s = torch.empty((E, rows, cols // 32), dtype=torch.uint8, device=device)
        fill_packed(p, synth.stream_key(spec.seed, layer, tp))
        fill_scales(s, synth.stream_key(spec.seed, layer, ts))
        d[name + "_packed"] = p
        d[name + "_scales"] = s
    sh = synth.make_shared(spec, layer)
    if sh is None:
        d["sh_gate"] = d["sh_up"] = d["sh_down"] = None
    else:
        d["sh_gate"], d["sh_up"], d["sh_down"] = (bf16_tensor(s, device) for s in sh)
    lat = synth.make_latent(spec, layer)
    if lat is None:
        d["lat_down"] = d["lat_up"] = d["lat_norm"] = None
    else:
        d["lat_down"], d["lat_up"] = bf16_tensor(lat[0], device), bf16_tensor(lat[1], device)
        d["lat_norm"] = torch.from_numpy(lat[2]).to(device)
    return d


def make_layer(spec: synth.LayerSpec, tensors):
    """A library Layer over the tensors of ``layer_tensors``."""
    import mxfp4_routed_expert_sigmoid_amd as k3
    lat = spec.latent > 0
    cfg = k3.make_config(spec.hidden, spec.inter, spec.n_experts, spec.topk, spec.shared_inter,
                         spec.renorm, spec.routed_scale, spec.act, spec.situ_b1, spec.situ_b2,
                         spec.latent, spec.latent_norm if lat else 0, spec.rms_eps if lat else 0.0)
    t = tensors
    return k3.Layer(cfg, t["router_w"], t["router_bias"], t["gate_packed"], t["gate_scales"],
                    t["up_packed"], t["up_scales"], t["down_packed"], t["down_scales"],
                    t["sh_gate"], t["sh_up"], t["sh_down"], t.get("lat_down"), t.get("lat_up"),
                    t.get("lat_norm") if lat and spec.latent_norm else None)
