"""Python binding of libk3moe, the MI355X sigmoid-routed MXFP4 expert layer.

Argument marshalling only: every step of the layer runs in the library's
gfx950 kernels (``csrc/``); PyTorch supplies device buffers and the stream.
The C ABI is declared in ``include/k3moe.h``; the names here mirror it.
If the library has not been built this module raises ImportError: there is
no fallback path.
"""
import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libk3moe.so")

ABI_VERSION = 3
ACT_SITU, ACT_SWIGLU = 1, 2

STATUS = {0: "ok", 1: "invalid argument", 2: "invalid or incomplete config",
          3: "unsupported shape", 4: "pointer or stride not aligned",
          5: "workspace missing, misaligned or too small", 6: "out of device memory",
          7: "HIP runtime error"}


class K3MoeError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {STATUS.get(status, status)} (status {status})")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("abi_version", ctypes.c_uint32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("renorm", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("act", ctypes.c_int32),
                ("situ_b1", ctypes.c_float), ("situ_b2", ctypes.c_float),
                ("latent", ctypes.c_int32), ("latent_norm", ctypes.c_int32),
                ("rms_eps", ctypes.c_float)]


class MXFP4(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("expert_stride_packed", ctypes.c_int64),
                ("expert_stride_scales", ctypes.c_int64)]


class Weights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", MXFP4), ("up", MXFP4), ("down", MXFP4),
                ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p),
                ("sh_down", ctypes.c_void_p), ("lat_down", ctypes.c_void_p),
                ("lat_up", ctypes.c_void_p), ("lat_norm", ctypes.c_void_p)]


class CacheStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("steps", "requests", "resident_hits", "misses",
                                                "evictions", "dropped", "bytes_read")]


_lib = None
EXPORTS = ("k3moe_layer_create", "k3moe_workspace_size", "k3moe_route", "k3moe_forward",
           "k3moe_route_forward", "k3moe_forward_noalloc", "k3moe_forward_residual", "k3moe_step",
           "k3moe_cache_create", "k3moe_cache_device_bytes", "k3moe_cache_workspace_size",
           "k3moe_cache_forward", "k3moe_cache_stats_read", "k3moe_cache_slots", "k3moe_cache_reset", "k3moe_cache_destroy",
           "k3moe_error_count", "k3moe_error_reset", "k3moe_profile_enable",
           "k3moe_profile_read", "k3moe_layer_destroy", "k3moe_status_string")
STAGES = ("router", "topk", "perm", "gateup", "shared_gateup", "down", "combine",
          "latent_in", "latent_out", "prenorm", "cache_plan", "cache_fill", "gateup_tiles",
          "down_tiles")


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
        L.k3moe_layer_create.restype = st
        L.k3moe_layer_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights),
                                         ctypes.POINTER(P)]
        L.k3moe_workspace_size.restype = st
        L.k3moe_workspace_size.argtypes = [P, i32, ctypes.POINTER(ctypes.c_size_t)]
        L.k3moe_route.restype = st
        L.k3moe_route.argtypes = [P, P, i32, P, P, P, P, ctypes.c_size_t, P]
        L.k3moe_forward.restype = st
        L.k3moe_forward.argtypes = [P, P, i32, P, P, P, P, ctypes.c_size_t, P]
        L.k3moe_route_forward.restype = st
        L.k3moe_route_forward.argtypes = [P, P, i32, P, P, P, P, P, ctypes.c_size_t, P]
        L.k3moe_forward_noalloc.restype = st
        L.k3moe_forward_noalloc.argtypes = [P, P, i32, P, P, P, P]
        L.k3moe_forward_residual.restype = st
        L.k3moe_forward_residual.argtypes = [P, P, i32, P, P, P, P, P, ctypes.c_size_t, P]
        L.k3moe_step.restype = st
        L.k3moe_step.argtypes = [P, P, i32, P, ctypes.c_float, P, P, P, P, P, ctypes.c_size_t, P]
        L.k3moe_cache_create.restype = st
        L.k3moe_cache_create.argtypes = [P, i32, ctypes.POINTER(P)]
        L.k3moe_cache_device_bytes.restype = st
        L.k3moe_cache_device_bytes.argtypes = [P, i32, ctypes.POINTER(ctypes.c_size_t)]
        L.k3moe_cache_workspace_size.restype = st
        L.k3moe_cache_workspace_size.argtypes = [P, i32, ctypes.POINTER(ctypes.c_size_t)]
        L.k3moe_cache_forward.restype = st
        L.k3moe_cache_forward.argtypes = [P, P, i32, P, P, P, P, ctypes.c_size_t, P]
        L.k3moe_cache_stats_read.restype = st
        L.k3moe_cache_stats_read.argtypes = [P, ctypes.POINTER(CacheStats), P]
        L.k3moe_cache_slots.restype = st
        L.k3moe_cache_slots.argtypes = [P, P, P]
        L.k3moe_cache_reset.restype = st
        L.k3moe_cache_reset.argtypes = [P, P]
        L.k3moe_cache_destroy.restype = None
        L.k3moe_cache_destroy.argtypes = [P]
        L.k3moe_error_count.restype = st
        L.k3moe_error_count.argtypes = [P, ctypes.POINTER(ctypes.c_uint64), P]
        L.k3moe_error_reset.restype = st
        L.k3moe_error_reset.argtypes = [P, P]
        L.k3moe_profile_enable.restype = st
        L.k3moe_profile_enable.argtypes = [P, st]
        L.k3moe_profile_read.restype = st
        L.k3moe_profile_read.argtypes = [P, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_int64), i32, P]
        L.k3moe_layer_destroy.restype = None
        L.k3moe_layer_destroy.argtypes = [P]
        L.k3moe_status_string.restype = ctypes.c_char_p
        L.k3moe_status_string.argtypes = [st]
        _lib = L
    return _lib


def make_config(hidden, inter, n_experts, topk, shared_inter=0, renorm=1, routed_scale=1.0,
                act=ACT_SITU, situ_b1=4.0, situ_b2=25.0, latent=0, latent_norm=0, rms_eps=0.0):
    return Config(ctypes.sizeof(Config), ABI_VERSION, hidden, inter, n_experts, topk,
                  shared_inter, renorm, routed_scale, act, situ_b1, situ_b2, latent,
                  latent_norm, rms_eps)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, device):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, what):
    if status != 0:
        raise K3MoeError(status, what)


def _shape(t, shape, name):
    """Refuse a tensor whose shape is not `shape` (None: absent, accepted).
    The C ABI takes raw pointers, so a mis-shaped tensor would become an
    out-of-bounds device access; it is refused here before any call."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _rows(x, width, name="x"):
    """Token count of a [T][width] tensor (refused otherwise)."""
    if x.dim() != 2 or x.shape[1] != width:
        raise ValueError(f"{name}: shape {tuple(x.shape)}, expected [T][{width}]")
    return x.shape[0]


def _dev(t, dtype_sizes, name, pinned_ok=False):
    if t is None:
        return
    if not (t.is_cuda or (pinned_ok and t.is_pinned())):
        raise ValueError(f"{name} must be a device tensor" + (" or pinned host memory" if pinned_ok else ""))
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.element_size() not in dtype_sizes:
        raise ValueError(f"{name}: element size {t.element_size()} not in {dtype_sizes}")


class Layer:
    """A k3moe layer handle over caller-owned device weights.

    Weights (device tensors, contiguous): router_w bf16/int16 [E][H];
    router_bias fp32 [E] or None; gate/up packed uint8 [E][I][H/2] and scales
    uint8 [E][I][H/32]; down packed [E][H][I/2] and scales [E][H][I/32];
    shared sh_gate/sh_up [Is][H], sh_down [H][Is] (bf16/int16) or None.
    Latent layer (cfg.latent = L > 0): the experts are [E][I][L/2] (gate, up)
    and [E][L][I/2] (down), lat_down bf16 [L][H], lat_up bf16 [H][L],
    lat_norm fp32 [L] (None without the norm).
    The routed expert tensors may instead be pinned host tensors
    (pin_memory=True) for a layer served through a ``Cache``.
    The handle keeps references to the tensors so they outlive it.
    """

    def __init__(self, cfg: Config, router_w, router_bias, gate_packed, gate_scales, up_packed,
                 up_scales, down_packed, down_scales, sh_gate=None, sh_up=None, sh_down=None,
                 lat_down=None, lat_up=None, lat_norm=None):
        for t, n in ((router_w, "router_w"), (sh_gate, "sh_gate"), (sh_up, "sh_up"),
                     (sh_down, "sh_down"), (lat_down, "lat_down"), (lat_up, "lat_up")):
            _dev(t, (2,), n)
        _dev(router_bias, (4,), "router_bias")
        _dev(lat_norm, (4,), "lat_norm")
        for t, n in ((gate_packed, "gate_packed"), (gate_scales, "gate_scales"),
                     (up_packed, "up_packed"), (up_scales, "up_scales"),
                     (down_packed, "down_packed"), (down_scales, "down_scales")):
            _dev(t, (1,), n, pinned_ok=True)
        self.cfg = cfg
        self.device = router_w.device
        self._keep = (router_w, router_bias, gate_packed, gate_scales, up_packed, up_scales,
                      down_packed, down_scales, sh_gate, sh_up, sh_down, lat_down, lat_up, lat_norm)
        E = cfg.n_experts

        def mx(p, s):
            return MXFP4(p.data_ptr(), s.data_ptr(), p.numel() // E, s.numel() // E)

        self.weights = Weights(router_w.data_ptr(), _ptr(router_bias),
                               mx(gate_packed, gate_scales), mx(up_packed, up_scales),
                               mx(down_packed, down_scales), _ptr(sh_gate), _ptr(sh_up),
                               _ptr(sh_down), _ptr(lat_down), _ptr(lat_up), _ptr(lat_norm))
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(lib().k3moe_layer_create(ctypes.byref(cfg), ctypes.byref(self.weights),
                                            ctypes.byref(h)), "k3moe_layer_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            lib().k3moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, max_tokens: int) -> int:
        n = ctypes.c_size_t()
        _check(lib().k3moe_workspace_size(self.handle, int(max_tokens), ctypes.byref(n)),
               "k3moe_workspace_size")
        return n.value

    def workspace(self, max_tokens: int):
        """A device byte tensor big enough for max_tokens tokens (256-aligned)."""
        return torch.empty(self.workspace_size(max_tokens) + 256, dtype=torch.uint8,
                           device=self.device)

    @staticmethod
    def _ws(ws):
        base = ws.data_ptr()
        off = (-base) % 256
        return ctypes.c_void_p(base + off), ws.numel() - off

    def _call_ws(self, workspace, T, stream):
        """The caller's workspace, or a new one for T tokens. A new one is
        allocated on the current stream; when the call runs on another
        stream it is marked as used there, so the caching allocator does not
        hand its memory out again while the queued kernels still use it."""
        if workspace is not None:
            return workspace
        ws = self.workspace(T)
        if stream is not None and stream != torch.cuda.current_stream(self.device):
            ws.record_stream(stream)
        return ws

    def _check_tokens(self, T, **t):
        H, K, E = self.cfg.hidden, self.cfg.topk, self.cfg.n_experts
        shapes = {"idx": (T, K), "w": (T, K), "out": (T, H), "h": (T, H), "hb": (T, H),
                  "x_out": (T, H), "logits": (T, E), "gamma": (H,)}
        for name, tensor in t.items():
            _shape(tensor, shapes[name], name)

    def route(self, x, idx, w, logits=None, workspace=None, stream=None):
        """k3moe_route: x bf16 [T][H] -> idx int32 [T][k], w fp32 [T][k] (written)."""
        T = _rows(x, self.cfg.hidden)
        self._check_tokens(T, idx=idx, w=w, logits=logits)
        _dev(x, (2,), "x"), _dev(idx, (4,), "idx"), _dev(w, (4,), "w"), _dev(logits, (4,), "logits")
        ws = self._call_ws(workspace, T, stream)
        p, n = self._ws(ws)
        _check(lib().k3moe_route(self.handle, x.data_ptr(), T, idx.data_ptr(), w.data_ptr(),
                                 _ptr(logits), p, n, _stream(stream, self.device)), "k3moe_route")

    def forward(self, x, idx, w, out, workspace=None, stream=None):
        """k3moe_forward: out fp32 [T][H] (written) from x, idx, w."""
        T = _rows(x, self.cfg.hidden)
        self._check_tokens(T, idx=idx, w=w, out=out)
        _dev(x, (2,), "x"), _dev(idx, (4,), "idx"), _dev(w, (4,), "w"), _dev(out, (4,), "out")
        ws = self._call_ws(workspace, T, stream)
        p, n = self._ws(ws)
        _check(lib().k3moe_forward(self.handle, x.data_ptr(), T, idx.data_ptr(), w.data_ptr(),
                                   out.data_ptr(), p, n, _stream(stream, self.device)),
               "k3moe_forward")

    def route_forward(self, x, idx, w, out, logits=None, workspace=None, stream=None):
        """k3moe_route_forward: route x, then the expert layer on those routes;
        idx int32 [T][k], w fp32 [T][k] and out fp32 [T][H] written."""
        T = _rows(x, self.cfg.hidden)
        self._check_tokens(T, idx=idx, w=w, out=out, logits=logits)
        _dev(x, (2,), "x"), _dev(idx, (4,), "idx"), _dev(w, (4,), "w"), _dev(out, (4,), "out")
        _dev(logits, (4,), "logits")
        ws = self._call_ws(workspace, T, stream)
        p, n = self._ws(ws)
        _check(lib().k3moe_route_forward(self.handle, x.data_ptr(), T, idx.data_ptr(), w.data_ptr(),
                                         _ptr(logits), out.data_ptr(), p, n, _stream(stream, self.device)),
               "k3moe_route_forward")

    def forward_noalloc(self, x, idx, w, out, stream=None):
        """k3moe_forward_noalloc: k3moe_forward on the library's fixed per-GPU
        scratch array (no workspace, nothing allocated); calls on one GPU must
        not overlap."""
        T = _rows(x, self.cfg.hidden)
        self._check_tokens(T, idx=idx, w=w, out=out)
        _dev(x, (2,), "x"), _dev(idx, (4,), "idx"), _dev(w, (4,), "w"), _dev(out, (4,), "out")
        _check(lib().k3moe_forward_noalloc(self.handle, x.data_ptr(), T, idx.data_ptr(), w.data_ptr(),
                                           out.data_ptr(), _stream(stream, self.device)),
               "k3moe_forward_noalloc")

    def forward_residual(self, x, idx, w, h, hb=None, workspace=None, stream=None):
        """k3moe_forward_residual: h fp32 [T][H] += forward(x, idx, w), in place;
        hb (bf16 [T][H], optional, may be x) receives bf16 of the updated h."""
        T = _rows(x, self.cfg.hidden)
        self._check_tokens(T, idx=idx, w=w, h=h, hb=hb)
        _dev(x, (2,), "x"), _dev(idx, (4,), "idx"), _dev(w, (4,), "w"), _dev(h, (4,), "h"), _dev(hb, (2,), "hb")
        ws = self._call_ws(workspace, T, stream)
        p, n = self._ws(ws)
        _check(lib().k3moe_forward_residual(self.handle, x.data_ptr(), T, idx.data_ptr(), w.data_ptr(),
                                            h.data_ptr(), _ptr(hb), p, n, _stream(stream, self.device)),
               "k3moe_forward_residual")

    def step(self, h, gamma, eps, idx, w, x_out=None, hb=None, workspace=None, stream=None):
        """k3moe_step: h fp32 [T][H] += layer(bf16(RMSNorm(h) * gamma)), in place;
        idx int32 [T][k] and w fp32 [T][k] written; x_out / hb (bf16 [T][H],
        optional) receive the normed input and bf16 of the updated h."""
        T = _rows(h, self.cfg.hidden, "h")
        self._check_tokens(T, gamma=gamma, idx=idx, w=w, x_out=x_out, hb=hb)
        _dev(h, (4,), "h"), _dev(gamma, (4,), "gamma"), _dev(idx, (4,), "idx"), _dev(w, (4,), "w")
        _dev(x_out, (2,), "x_out"), _dev(hb, (2,), "hb")
        ws = self._call_ws(workspace, T, stream)
        p, n = self._ws(ws)
        _check(lib().k3moe_step(self.handle, h.data_ptr(), T, gamma.data_ptr(), float(eps),
                                _ptr(x_out), idx.data_ptr(), w.data_ptr(), _ptr(hb), p, n,
                                _stream(stream, self.device)), "k3moe_step")

    def error_count(self, stream=None) -> int:
        n = ctypes.c_uint64()
        _check(lib().k3moe_error_count(self.handle, ctypes.byref(n), _stream(stream, self.device)),
               "k3moe_error_count")
        return n.value

    def profile(self, enable: bool):
        """Turn per-stage event timing on or off (k3moe_profile_enable)."""
        _check(lib().k3moe_profile_enable(self.handle, int(bool(enable))), "k3moe_profile_enable")

    def profile_read(self, stream=None):
        """{stage: (total_ms, launches)} since the last read (k3moe_profile_read)."""
        n = len(STAGES)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        _check(lib().k3moe_profile_read(self.handle, ms, cnt, n, _stream(stream, self.device)),
               "k3moe_profile_read")
        return {STAGES[i]: (ms[i], cnt[i]) for i in range(n)}

    def error_reset(self, stream=None):
        _check(lib().k3moe_error_reset(self.handle, _stream(stream, self.device)),
               "k3moe_error_reset")


def cache_device_bytes(cfg: Config, n_slots: int) -> int:
    """Device bytes a cache of n_slots slots allocates for a layer of this
    config (k3moe_cache_device_bytes; no device call)."""
    n = ctypes.c_size_t()
    _check(lib().k3moe_cache_device_bytes(ctypes.byref(cfg), int(n_slots), ctypes.byref(n)),
           "k3moe_cache_device_bytes")
    return n.value


class Cache:
    """An HBM arena of n_slots expert slots in front of a layer whose routed
    experts live in pinned host memory (k3moe_cache_*). Keeps the layer alive."""

    def __init__(self, layer: Layer, n_slots: int):
        self.layer = layer
        self.device = layer.device
        self.n_slots = int(n_slots)
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(lib().k3moe_cache_create(layer.handle, self.n_slots, ctypes.byref(h)),
                   "k3moe_cache_create")
        self.handle = h

    def workspace_size(self, max_tokens: int) -> int:
        n = ctypes.c_size_t()
        _check(lib().k3moe_cache_workspace_size(self.handle, int(max_tokens), ctypes.byref(n)),
               "k3moe_cache_workspace_size")
        return n.value

    def workspace(self, max_tokens: int):
        return torch.empty(self.workspace_size(max_tokens) + 256, dtype=torch.uint8,
                           device=self.device)

    def forward(self, x, idx, w, out, workspace=None, stream=None):
        """k3moe_cache_forward: out fp32 [T][H] (written) through the slots."""
        T = _rows(x, self.layer.cfg.hidden)
        self.layer._check_tokens(T, idx=idx, w=w, out=out)
        _dev(x, (2,), "x"), _dev(idx, (4,), "idx"), _dev(w, (4,), "w"), _dev(out, (4,), "out")
        ws = workspace
        if ws is None:
            ws = self.workspace(T)
            if stream is not None and stream != torch.cuda.current_stream(self.device):
                ws.record_stream(stream)
        p, n = Layer._ws(ws)
        _check(lib().k3moe_cache_forward(self.handle, x.data_ptr(), T, idx.data_ptr(), w.data_ptr(),
                                         out.data_ptr(), p, n, _stream(stream, self.device)),
               "k3moe_cache_forward")

    def stats(self, stream=None) -> dict:
        st = CacheStats()
        _check(lib().k3moe_cache_stats_read(self.handle, ctypes.byref(st), _stream(stream, self.device)),
               "k3moe_cache_stats_read")
        return {n: getattr(st, n) for n, _ in CacheStats._fields_}

    def slots(self, stream=None):
        """Expert held by each slot (-1: empty), as a list."""
        buf = (ctypes.c_int32 * self.n_slots)()
        _check(lib().k3moe_cache_slots(self.handle, buf, _stream(stream, self.device)),
               "k3moe_cache_slots")
        return list(buf)

    def reset(self, stream=None):
        _check(lib().k3moe_cache_reset(self.handle, _stream(stream, self.device)), "k3moe_cache_reset")

    def close(self):
        if getattr(self, "handle", None):
            lib().k3moe_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
