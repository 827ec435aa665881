"""GPU parity of the latent layer (experts between a bf16 down- and
up-projection, RMSNorm on the aggregate, shared expert on the original x)
through the C ABI, against the fp64 oracle.

Every input is seeded and synthetic (``synth``); expected values come only
from ``oracle``."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import REL_TOL, certify_rows, check_route, oracle_forward, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _layer(spec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import synth.device as sd
    t = sd.layer_tensors(spec, 0, DEV)
    return t, sd.make_layer(spec, t)


def _run(spec, layer, T, tokens=None):
    import synth.device as sd
    x_np = synth.make_x(spec, T)
    Wr, bias = synth.make_router(spec), synth.make_bias(spec)
    idx_r, w_r, _, ch = certify_rows(spec, x_np, Wr, bias)
    x = sd.bf16_tensor(x_np, DEV)
    idx = torch.empty((T, spec.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((T, spec.topk), dtype=torch.float32, device=DEV)
    layer.route(x, idx, w)
    torch.cuda.synchronize()
    assert check_route(idx.cpu().numpy(), w.cpu().numpy(), idx_r, w_r, ch, spec.topk) == T
    out = torch.empty((T, spec.hidden), dtype=torch.float32, device=DEV)
    layer.forward(x, torch.from_numpy(idx_r).to(DEV), torch.from_numpy(w_r).to(DEV), out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    ref, denom, drops = oracle_forward(spec, x_np, idx_r, w_r, tokens=tokens)
    assert drops == 0
    err = rel_err(o[tokens], ref, denom)
    print(f"[latent] T={T} max rel err {err:.3g}", flush=True)
    assert err <= REL_TOL
    return o, x_np, idx_r, w_r


@pytest.mark.parametrize("T", [1, 2, 5, 17, 40, 129])
def test_tiny_latent(T):
    # hidden 256, latent 128: every expert takes the grouped GEMM tiles
    spec = synth.LayerSpec(hidden=256, inter=128, n_experts=8, topk=2, shared_inter=128,
                           bias_std=0.05, seed=90 + T, latent=128)
    _, layer = _layer(spec)
    _run(spec, layer, T)


@pytest.mark.parametrize("T", [1, 7])
def test_tiny_latent_without_norm_or_shared(T):
    # T = 1 takes the one-token projections (no norm: the aggregate as is)
    spec = synth.LayerSpec(hidden=256, inter=128, n_experts=8, topk=2, shared_inter=0,
                           bias_std=0.05, seed=97, latent=256, latent_norm=0)
    _, layer = _layer(spec)
    _run(spec, layer, T)


@pytest.mark.parametrize("T,routing", [(1, "normal"), (5, "normal"), (40, "normal"), (129, "zipf"),
                                       (300, "zipf")])
def test_mid_latent_stream_and_gemm(T, routing):
    # hidden 1024, latent 512: light experts stream, heavy ones take GEMM tiles
    spec = synth.LayerSpec(hidden=1024, inter=512, n_experts=16, topk=4, shared_inter=512,
                           bias_std=0.05, routing=routing, seed=100 + T, latent=512)
    _, layer = _layer(spec)
    o, x_np, idx_r, w_r = _run(spec, layer, T)
    if T >= 129:
        # deterministic: a second call gives the same bits
        import synth.device as sd
        x = sd.bf16_tensor(x_np, DEV)
        out = torch.empty((T, spec.hidden), dtype=torch.float32, device=DEV)
        layer.forward(x, torch.from_numpy(idx_r).to(DEV), torch.from_numpy(w_r).to(DEV), out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), o)


_PAGES = {}


def _pages():
    if "l" not in _PAGES:
        import test_gpu_layer
        test_gpu_layer._FULL.clear()
        torch.cuda.empty_cache()
        spec = synth.pages_latent_spec(seed=0)
        _PAGES["l"] = (spec,) + _layer(spec)
    return _PAGES["l"]


def test_pages_latent_decode_T1():
    spec, _, layer = _pages()
    _run(spec, layer, 1)


def test_pages_latent_T64_all_tokens():
    spec, _, layer = _pages()
    _run(spec, layer, 64)


def test_pages_latent_release():
    _PAGES.clear()
    torch.cuda.empty_cache()
