"""fp64 CPU oracle of the sigmoid-routed MXFP4 expert layer (ctypes wrapper).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The product path
never does, and the two share no code.

Every function follows the "kimi-k3-in-c" README: §4 (MXFP4 format and the
matrix-vector product over nibbles), §5 (bf16 widening, k3_rmsnorm), §9
(k3_router, k3_moe with and without its latent projections, k3_situ_glu).
The arithmetic lives in ``k3moe_oracle.c``; this module only marshals numpy
arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

ACT_SITU = 1
ACT_SWIGLU = 2

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.k3o_e2m1.restype = ctypes.c_double
        L.k3o_e2m1.argtypes = [ctypes.c_int]
        L.k3o_e8m0.restype = ctypes.c_double
        L.k3o_e8m0.argtypes = [ctypes.c_int]
        L.k3o_bf16.restype = ctypes.c_double
        L.k3o_bf16.argtypes = [ctypes.c_uint16]
        L.k3o_act.restype = ctypes.c_double
        L.k3o_act.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int,
                              ctypes.c_double, ctypes.c_double]
        L.k3o_mxfp4_gemv.restype = None
        L.k3o_mxfp4_gemv.argtypes = [P, P, P, P, P, i64, i64]
        L.k3o_bf16_gemv.restype = None
        L.k3o_bf16_gemv.argtypes = [P, P, P, P, i64, i64]
        L.k3o_route.restype = ctypes.c_int
        L.k3o_route.argtypes = [P, P, P, P, P, P, P, i64, i64, i64, i64,
                                ctypes.c_int, ctypes.c_float]
        L.k3o_forward.restype = i64
        L.k3o_forward.argtypes = [P, P, P, i64, i64, i64, P, P, i64, i64, P,
                                  P, P, P, P, P, P, P, P, P, i64,
                                  ctypes.c_int, ctypes.c_double, ctypes.c_double]
        L.k3o_rmsnorm.restype = ctypes.c_double
        L.k3o_rmsnorm.argtypes = [P, P, P, i64, ctypes.c_double]
        L.k3o_forward_latent.restype = i64
        L.k3o_forward_latent.argtypes = [P, P, P, i64, i64, i64, i64, P, P, i64, i64, P,
                                         P, P, P, P, P, P, P, P, ctypes.c_int, P, ctypes.c_double,
                                         P, P, P, i64, ctypes.c_int, ctypes.c_double, ctypes.c_double]
        L.k3o_bf16_rne.restype = ctypes.c_uint16
        L.k3o_bf16_rne.argtypes = [ctypes.c_float]
        L.k3o_prenorm_bf16.restype = None
        L.k3o_prenorm_bf16.argtypes = [P, P, P, i64, i64, ctypes.c_float]
        L.k3o_threads.restype = ctypes.c_int
        L.k3o_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def e2m1(code: int) -> float:
    return lib().k3o_e2m1(int(code))


def e8m0(b: int) -> float:
    return lib().k3o_e8m0(int(b))


def bf16(h: int) -> float:
    return lib().k3o_bf16(int(h))


def act(g: float, u: float, kind: int = ACT_SITU, b1: float = 4.0, b2: float = 25.0) -> float:
    return lib().k3o_act(float(g), float(u), int(kind), float(b1), float(b2))


def threads() -> int:
    return lib().k3o_threads()


def mxfp4_gemv(x, packed, scales, K, rows, want_abs=False):
    """y = W x for an MXFP4 matrix W [rows][K]; x is fp64 [K]."""
    x = _c(x, np.float64)
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    assert x.size == K and packed.size == rows * ((K + 1) // 2)
    assert scales.size == rows * ((K + 31) // 32)
    y = np.empty(rows, np.float64)
    yabs = np.empty(rows, np.float64) if want_abs else None
    lib().k3o_mxfp4_gemv(_ptr(y), _ptr(yabs), _ptr(x), _ptr(packed), _ptr(scales), K, rows)
    return (y, yabs) if want_abs else y


def bf16_gemv(x, W, K, rows, want_abs=False):
    """y = W x for a bf16 matrix W [rows][K] (uint16 bit patterns); x is fp64."""
    x = _c(x, np.float64)
    W = _c(W, np.uint16)
    assert x.size == K and W.size == rows * K
    y = np.empty(rows, np.float64)
    yabs = np.empty(rows, np.float64) if want_abs else None
    lib().k3o_bf16_gemv(_ptr(y), _ptr(yabs), _ptr(x), _ptr(W), K, rows)
    return (y, yabs) if want_abs else y


def route(x, Wr, bias, topk, renorm=1, routed_scale=1.0, want_detail=False):
    """Router for x bf16 [T][H] and Wr bf16 [E][H] (uint16 patterns).

    Returns idx int32 [T][topk] and w float32 [T][topk]; with want_detail also
    the fp64 logits [T][E] and fp32 selection scores ch [T][E]."""
    x = _c(x, np.uint16)
    Wr = _c(Wr, np.uint16)
    T, H = x.shape
    E = Wr.shape[0]
    assert Wr.shape == (E, H)
    bias = _c(bias, np.float32)
    if bias is not None:
        assert bias.shape == (E,)
    idx = np.empty((T, topk), np.int32)
    w = np.empty((T, topk), np.float32)
    logits = np.empty((T, E), np.float64) if want_detail else None
    ch = np.empty((T, E), np.float32) if want_detail else None
    rc = lib().k3o_route(_ptr(idx), _ptr(w), _ptr(logits), _ptr(ch), _ptr(x), _ptr(Wr),
                         _ptr(bias), T, H, E, topk, int(renorm), float(routed_scale))
    if rc != 0:
        raise ValueError("oracle route: invalid sizes")
    if want_detail:
        return idx, w, logits, ch
    return idx, w


class ExpertSet:
    """Host copies of a subset of experts' MXFP4 matrices, keyed by expert id.

    gate/up packed [n][I][H/2] and scales [n][I][H/32]; down packed [n][H][I/2]
    and scales [n][H][I/32]; ``experts`` lists the expert id held in each slot.
    """

    def __init__(self, experts, n_experts, gate_packed, gate_scales, up_packed,
                 up_scales, down_packed, down_scales):
        self.experts = np.asarray(experts, np.int64)
        self.slot_of = np.full(n_experts, -1, np.int32)
        for s, e in enumerate(self.experts):
            self.slot_of[e] = s
        self.n_experts = n_experts
        self.gate_packed = _c(gate_packed, np.uint8)
        self.gate_scales = _c(gate_scales, np.uint8)
        self.up_packed = _c(up_packed, np.uint8)
        self.up_scales = _c(up_scales, np.uint8)
        self.down_packed = _c(down_packed, np.uint8)
        self.down_scales = _c(down_scales, np.uint8)


def forward(x, idx, w, experts: ExpertSet, H, I, shared=None, act_kind=ACT_SITU,
            b1=4.0, b2=25.0, want_denom=True):
    """Layer output (fp64 [T][H]) and per-element error denominators.

    ``shared`` is None or a tuple (S1 [Is][H], S3 [Is][H], S2 [H][Is]) of bf16
    uint16 patterns. Returns (out, denom, drops)."""
    x = _c(x, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    T = x.shape[0]
    topk = idx.shape[1]
    assert x.shape == (T, H) and idx.shape == (T, topk) and w.shape == (T, topk)
    ns = experts.experts.size
    assert experts.gate_packed.size == ns * I * ((H + 1) // 2)
    assert experts.gate_scales.size == ns * I * ((H + 31) // 32)
    assert experts.down_packed.size == ns * H * ((I + 1) // 2)
    assert experts.down_scales.size == ns * H * ((I + 31) // 32)
    if shared is not None:
        S1, S3, S2 = (_c(s, np.uint16) for s in shared)
        Is = S1.shape[0]
        assert S1.shape == (Is, H) and S3.shape == (Is, H) and S2.shape == (H, Is)
    else:
        S1 = S3 = S2 = None
        Is = 0
    out = np.empty((T, H), np.float64)
    denom = np.empty((T, H), np.float64) if want_denom else None
    drops = lib().k3o_forward(
        _ptr(out), _ptr(denom), _ptr(x), T, H, I, _ptr(idx), _ptr(w), topk,
        experts.n_experts, _ptr(experts.slot_of),
        _ptr(experts.gate_packed), _ptr(experts.gate_scales),
        _ptr(experts.up_packed), _ptr(experts.up_scales),
        _ptr(experts.down_packed), _ptr(experts.down_scales),
        _ptr(S1), _ptr(S3), _ptr(S2), Is, int(act_kind), float(b1), float(b2))
    if drops < 0:
        raise ValueError("oracle forward: a selected expert has no slot, or bad sizes")
    return out, denom, int(drops)


def rmsnorm(v, gamma=None, eps=1e-5):
    """RMSNorm of an fp64 vector (epsilon inside the square root); returns
    (out, inv)."""
    v = _c(v, np.float64)
    gamma = _c(gamma, np.float32)
    if gamma is not None:
        assert gamma.size == v.size
    out = np.empty_like(v)
    inv = lib().k3o_rmsnorm(_ptr(out), _ptr(v), _ptr(gamma), v.size, float(eps))
    return out, inv


def bf16_rne(v: float) -> int:
    """fp32 value -> bf16 bits, nearest with ties to even (by the definition)."""
    return int(lib().k3o_bf16_rne(float(np.float32(v))))


def prenorm_bf16(h, gamma, eps):
    """The pre-MoE norm of a decoder layer, rounded to bf16: uint16 [T][n]
    from fp32 h [T][n] and gain fp32 [n] (k3_rmsnorm's float form)."""
    h = _c(h, np.float32)
    gamma = _c(gamma, np.float32)
    T, n = h.shape
    assert gamma.shape == (n,)
    x = np.empty((T, n), np.uint16)
    lib().k3o_prenorm_bf16(_ptr(x), _ptr(h), _ptr(gamma), T, n, float(np.float32(eps)))
    return x


def forward_latent(x, idx, w, experts: ExpertSet, H, L, I, lat_down, lat_up, norm=True,
                   gamma=None, eps=1e-5, shared=None, act_kind=ACT_SITU, b1=4.0, b2=25.0,
                   want_denom=True):
    """Latent layer output (fp64 [T][H]), error denominators and drops.

    Experts are at width L: gate/up [I][L], down [L][I]. lat_down bf16 [L][H],
    lat_up bf16 [H][L]; gamma fp32 [L] (norm only); shared as in ``forward``."""
    x = _c(x, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    T = x.shape[0]
    topk = idx.shape[1]
    assert x.shape == (T, H) and idx.shape == (T, topk) and w.shape == (T, topk)
    ns = experts.experts.size
    assert experts.gate_packed.size == ns * I * ((L + 1) // 2)
    assert experts.gate_scales.size == ns * I * ((L + 31) // 32)
    assert experts.down_packed.size == ns * L * ((I + 1) // 2)
    assert experts.down_scales.size == ns * L * ((I + 31) // 32)
    Wd = _c(lat_down, np.uint16)
    Wu = _c(lat_up, np.uint16)
    assert Wd.shape == (L, H) and Wu.shape == (H, L)
    gamma = _c(gamma, np.float32)
    if norm and gamma is not None:
        assert gamma.shape == (L,)
    if shared is not None:
        S1, S3, S2 = (_c(s, np.uint16) for s in shared)
        Is = S1.shape[0]
        assert S1.shape == (Is, H) and S3.shape == (Is, H) and S2.shape == (H, Is)
    else:
        S1 = S3 = S2 = None
        Is = 0
    out = np.empty((T, H), np.float64)
    denom = np.empty((T, H), np.float64) if want_denom else None
    drops = lib().k3o_forward_latent(
        _ptr(out), _ptr(denom), _ptr(x), T, H, L, I, _ptr(idx), _ptr(w), topk,
        experts.n_experts, _ptr(experts.slot_of),
        _ptr(experts.gate_packed), _ptr(experts.gate_scales),
        _ptr(experts.up_packed), _ptr(experts.up_scales),
        _ptr(experts.down_packed), _ptr(experts.down_scales),
        _ptr(Wd), _ptr(Wu), int(bool(norm)), _ptr(gamma), float(eps),
        _ptr(S1), _ptr(S3), _ptr(S2), Is, int(act_kind), float(b1), float(b2))
    if drops < 0:
        raise ValueError("oracle forward_latent: a selected expert has no slot, or bad sizes")
    return out, denom, int(drops)
