"""k3moe_forward_noalloc (the allocation-free variant of k3moe_forward, on the
library's fixed per-GPU scratch array) against k3moe_forward, through the C
ABI. Same kernels, so the outputs must be identical bit for bit; two calls in
a row, the second with a smaller batch, so a stale first call cannot hide."""
import numpy as np
import pytest
import torch

import mxfp4_routed_expert_sigmoid_amd as k3
import oracle
import synth
from gpu_helpers import REL_TOL, oracle_forward, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCRATCH_BYTES = 64 << 20


def _layer(spec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import synth.device as sd
    return sd.make_layer(spec, sd.layer_tensors(spec, 0, DEV)), sd


def _inputs(spec, sd, T, attempt):
    x_np = synth.make_x(spec, T, attempt=attempt)
    idx_r, w_r = oracle.route(x_np, synth.make_router(spec), synth.make_bias(spec), spec.topk)
    x = sd.bf16_tensor(x_np, DEV)
    idx = torch.from_numpy(np.ascontiguousarray(idx_r, np.int32)).to(DEV)
    w = torch.from_numpy(np.ascontiguousarray(w_r, np.float32)).to(DEV)
    return x_np, idx_r, w_r, x, idx, w


def _both(layer, x, idx, w, H):
    T = x.shape[0]
    ref = torch.empty((T, H), dtype=torch.float32, device=DEV)
    got = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    layer.forward(x, idx, w, ref)
    layer.forward_noalloc(x, idx, w, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("kind,Ts", [("mid", (40, 5)), ("mid", (129, 1)), ("tiny", (17, 2)),
                                     ("latent", (9, 1))])
def test_noalloc_matches_forward_two_calls(kind, Ts):
    if kind == "mid":   # streaming kernels and tile GEMMs, shared expert
        spec = synth.LayerSpec(hidden=512, inter=512, n_experts=16, topk=4, shared_inter=256,
                               bias_std=0.05, routing="zipf" if Ts[0] > 128 else "normal", seed=71)
    elif kind == "tiny":
        spec = synth.tiny_spec(seed=72)
    else:               # a latent layer: projections and the norm in the scratch too
        spec = synth.LayerSpec(hidden=512, inter=256, n_experts=8, topk=2, shared_inter=256,
                               bias_std=0.05, latent=256, latent_norm=1, rms_eps=1e-5, seed=73)
    layer, sd = _layer(spec)
    for call, T in enumerate(Ts):
        x_np, idx_r, w_r, x, idx, w = _inputs(spec, sd, T, attempt=call)
        ref, got = _both(layer, x, idx, w, spec.hidden)
        assert np.array_equal(got, ref), (kind, call, T)
        # and against the oracle, on the first tokens
        few = np.arange(min(T, 3))
        o, d, _ = oracle_forward(spec, x_np, idx_r, w_r, tokens=few)
        assert rel_err(got[few], o, d) <= REL_TOL


def test_noalloc_full_shape_decode_then_batch():
    spec = synth.full_spec(seed=74)
    layer, sd = _layer(spec)
    for call, T in enumerate((3, 1)):
        x_np, idx_r, w_r, x, idx, w = _inputs(spec, sd, T, attempt=call)
        ref, got = _both(layer, x, idx, w, spec.hidden)
        assert np.array_equal(got, ref), (call, T)


def test_noalloc_refuses_batches_beyond_the_scratch():
    spec = synth.tiny_spec(seed=75)
    layer, sd = _layer(spec)
    # the largest batch whose workspace fits the 64 MiB scratch, and one more
    lo, hi = 1, 1 << 20
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if layer.workspace_size(mid) <= SCRATCH_BYTES:
            lo = mid
        else:
            hi = mid - 1
    T_max = lo
    assert layer.workspace_size(T_max + 1) > SCRATCH_BYTES
    x = torch.zeros((T_max + 1, spec.hidden), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((T_max + 1, spec.topk), dtype=torch.int32, device=DEV)
    w = torch.zeros((T_max + 1, spec.topk), dtype=torch.float32, device=DEV)
    out = torch.full((T_max + 1, spec.hidden), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(k3.K3MoeError) as e:
        layer.forward_noalloc(x, idx, w, out)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing was launched
    # the largest batch that fits runs
    layer.forward_noalloc(x[:T_max], idx[:T_max], w[:T_max], out[:T_max])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out[:T_max]).all())
