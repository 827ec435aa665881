"""GPU parity through a stack of 8 full-shape layers (896 experts each, all
resident: ~126 GB of MXFP4), with residual adds between them.

Reading of the stacked workload: h_{l+1} = h_l + out_l in fp32, and layer l
takes bf16_RNE(h_l); both happen in each layer's last kernel
(k3moe_forward_residual). The oracle gets the same bf16 input the GPU wrote
(teacher forcing per layer), so a layer is judged on its own arithmetic: the
updated stream within 1e-4 of D plus the add's one fp32 rounding, the bf16
copy equal to the nearest-even rounding of the GPU's own stream. Every
token's route is certified on every layer (a first pass, which checks
nothing, finds the tokens whose route is not certified on some layer, and
their inputs are redrawn), so the GPU's ids equal the oracle's everywhere;
the forward is compared on the oracle's routes. Every input is seeded and
synthetic; expected values come only from ``oracle``."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (_REDRAW, _REDRAW_MAX, REL_TOL, bf16_rne_np, check_route, oracle_forward,
                         route_certificate)

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


def _pass(spec, layers, x0, check):
    """One pass through the stack from the bf16 tokens x0. The stream h stays
    on the device: each layer's forward adds its output into h and writes
    bf16(h), the next layer's input, in its last kernel. check(l) gives the
    tokens whose outputs layer l compares with the oracle (None: a pass that
    only finds uncertified tokens). Returns the set of tokens whose route is
    not certified on some layer (the pass stops at the first such layer)."""
    import synth.device as sd
    T = x0.shape[0]
    h0 = synth.bf16_to_f32(x0).astype(np.float32)
    h = torch.from_numpy(h0).to(DEV)
    xb = sd.bf16_tensor(x0, DEV)
    for l, (t, layer) in enumerate(layers):
        x_np = xb.view(torch.int16).cpu().numpy().view(np.uint16)
        h_old = h.cpu().numpy()
        Wr, bias = synth.make_router(spec, l), synth.make_bias(spec, l)
        idx_r, w_r, _, ch = oracle.route(x_np, Wr, bias, spec.topk, want_detail=True)
        bad = np.nonzero(~route_certificate(ch, spec.topk))[0]
        if bad.size:
            assert check is None, (l, bad)
            return set(bad.tolist())
        if check is not None:
            idx = torch.empty((T, spec.topk), dtype=torch.int32, device=DEV)
            w = torch.empty((T, spec.topk), dtype=torch.float32, device=DEV)
            layer.route(xb, idx, w)
            torch.cuda.synchronize()
            assert check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk) == T
        layer.forward_residual(xb, torch.from_numpy(idx_r.astype(np.int32)).to(DEV),
                               torch.from_numpy(w_r.astype(np.float32)).to(DEV), h, hb=xb)
        torch.cuda.synchronize()
        if check is None:
            continue
        h_new = h.cpu().numpy()
        sample = np.asarray(check(l))
        ref, denom, drops = oracle_forward(spec, x_np, idx_r, w_r, layer=l, tokens=sample)
        assert drops == 0
        want = h_old[sample].astype(np.float64) + ref
        bound = REL_TOL * denom * (1 + 2.0 ** -24) + 2.0 ** -24 * np.abs(want)
        ratio = float((np.abs(h_new[sample].astype(np.float64) - want) / bound).max())
        print(f"[stack] T={T} layer {l}: max err / bound {ratio:.3g} over {sample.size} tokens", flush=True)
        assert ratio <= 1.0
        assert np.array_equal(xb.view(torch.int16).cpu().numpy().view(np.uint16), bf16_rne_np(h_new))
    assert np.all(np.isfinite(h.cpu().numpy()))
    return set()


def _run(spec, layers, T, check):
    x0 = synth.make_x(spec, T, layer=0)
    for a in range(_REDRAW_MAX):
        bad = _pass(spec, layers, x0, None)
        if not bad:
            break
        for tok in sorted(bad):
            x0[tok] = synth.make_x(spec, 1, layer=0, attempt=_REDRAW + tok * _REDRAW_MAX + a)[0]
    else:
        raise AssertionError("a token stayed uncertified")
    _pass(spec, layers, x0, check)


def test_stack_8_layers_one_token(stack):
    spec, layers = stack
    _run(spec, layers, 1, lambda l: [0])


def test_stack_8_layers_16_tokens(stack):
    # every token compared on the first and the last layer, two on the others
    spec, layers = stack
    _run(spec, layers, 16, lambda l: range(16) if l in (0, N_LAYERS - 1) else [0, 11])
