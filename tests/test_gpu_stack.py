"""GPU parity through a stack of 8 full-shape layers (896 experts each, all
resident: ~126 GB of MXFP4), with residual adds between them.

Reading of the stacked workload: h_{l+1} = h_l + out_l in fp32, and layer l
takes bf16_RNE(h_l). The harness forms each layer's input from the GPU's own
residual stream and hands the same bf16 input to the oracle (teacher forcing
per layer), so a layer is judged on its own arithmetic; routes are checked per
layer (exact on certified tokens, a valid top-k within the certificate's
margin elsewhere) and the forward is compared on the oracle's routes. Every
input is seeded and synthetic; expected values come only from ``oracle``."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import REL_TOL, check_route, oracle_forward, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_LAYERS = 8


@pytest.fixture(scope="module")
def stack():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import synth.device as sd
    import test_gpu_layer
    test_gpu_layer._FULL.clear()  # free the single-layer cache first
    torch.cuda.empty_cache()
    spec = synth.full_spec(seed=0)
    layers = []
    for l in range(N_LAYERS):
        t = sd.layer_tensors(spec, l, DEV)
        layers.append((t, sd.make_layer(spec, t)))
    yield spec, layers
    for _, layer in layers:
        layer.close()
    layers.clear()
    torch.cuda.empty_cache()


def _run(spec, layers, T, sample):
    import synth.device as sd
    h = synth.bf16_to_f32(synth.make_x(spec, T, layer=0)).astype(np.float32)
    for l, (t, layer) in enumerate(layers):
        x_np = synth.bf16_bits(h)
        x = sd.bf16_tensor(x_np, DEV)
        Wr, bias = synth.make_router(spec, l), synth.make_bias(spec, l)
        idx = torch.empty((T, spec.topk), dtype=torch.int32, device=DEV)
        w = torch.empty((T, spec.topk), dtype=torch.float32, device=DEV)
        layer.route(x, idx, w)
        torch.cuda.synchronize()
        idx_r, w_r, _, ch = oracle.route(x_np, Wr, bias, spec.topk, want_detail=True)
        check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk)
        out = torch.empty((T, spec.hidden), dtype=torch.float32, device=DEV)
        layer.forward(x, torch.from_numpy(idx_r.astype(np.int32)).to(DEV),
                      torch.from_numpy(w_r.astype(np.float32)).to(DEV), out)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        ref, denom, drops = oracle_forward(spec, x_np, idx_r, w_r, layer=l, tokens=sample)
        assert drops == 0
        err = rel_err(o[sample], ref, denom)
        print(f"[stack] T={T} layer {l}: max rel err {err:.3g}", flush=True)
        assert err <= REL_TOL
        h = h + o
    assert np.all(np.isfinite(h))


def test_stack_8_layers_one_token(stack):
    spec, layers = stack
    _run(spec, layers, 1, [0])


def test_stack_8_layers_16_tokens(stack):
    spec, layers = stack
    _run(spec, layers, 16, [0, 11])
