#!/usr/bin/env python3
"""Benchmark of the sigmoid-routed MXFP4 expert layer on one MI355X.

One step = the whole hot path for one batch of synthetic tokens: route
(router GEMV, sigmoid + bias top-k) and forward (permutation for batches,
routed gate/up + activation, shared gate/up, down, shared down, router-order
combine), through the C ABI on one HIP stream. Inputs are
resident in HBM before the timed region starts.

Workloads (full shape: hidden 7168, 896 experts, top-16, inter 1536, one bf16
shared expert of inter 1536, bias N(0, 0.01)):
  decode   T = 1 token per step (default; the metric's configuration)
  batched  T = 64, uniformly random routing
  prefill  T = 2048, Zipf(1.1)-skewed routing
  latent   T = 1 (or --tokens) on the pages' latent layer: hidden 7168, experts in a 3584
           latent with inter 3072 (the same 17,547,264 B per expert), two
           shared experts of 3072 (one of 6144) on x, bf16 down- and
           up-projections, RMSNorm of the aggregate
  step     T = 1 through k3moe_step on the full shape: the decoder layer's
           pre-MoE RMSNorm of an fp32 residual stream into bf16 tokens, route,
           experts, the residual add fused into the last kernel
  stack    --layers (8) full-shape layers resident (126 GB), --tokens (1) per
           step through all of them on an fp32 residual stream, each layer a
           decoder-layer MoE step (k3moe_step: the pre-MoE RMSNorm with the
           layer's own gain, route with its own router, experts, the residual
           add in the last kernel); the norm keeps every layer's routes
           spread (a plain residual grows until the sigmoid scores saturate)
  cache    T = 1 (or --tokens) on the full shape with the 896 experts in pinned host memory
           and --slots of them in an HBM slot arena (k3moe_cache_forward):
           misses are read over the host link each step; --routing picks
           flat (normal) or Zipf(1.1) routes; reports the resident hit rate
Steps rotate over a pool of token batches so consecutive steps select
different experts (the 281 MB a decode step touches is not left in the
256 MB last-level cache by the previous step).

Prints one JSON line. ``value`` is routed-expert HBM GB/s: the algorithmic
bytes of the experts the step selects (17,547,264 B each, counted once per
distinct expert) over the whole step time. ``roofline`` is the dominant
kernel's algorithmic bytes per launch over its event-timed average duration
(measured in a second pass with per-stage events on), against 8 TB/s;
its ``traffic`` is the HBM bytes per dispatch that rocprofv3's counters
recorded for the same kernel source (profiles/), or null.
``cpu_baseline`` times the fp64 oracle on this host's cores on a bounded
sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-expert HBM GB/s (decode) and tokens/s per MoE layer, % of roofline"
HBM_PEAK_GBPS = 8000.0
HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction
STEP_EPS = 1e-5  # the pre-MoE norm's epsilon (the pages' rms_eps)
STREAM_MAX_TOKENS = 16  # experts with more assignments go to the tile GEMMs
BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA
MXFP4_PEAK_TFLOPS = 10100.0  # dense MXFP4 MFMA
FP8_PEAK_TFLOPS = 5000.0    # dense fp8 MFMA (the rate of an fp4 x fp8 scaled MFMA)
EXPERT_MATRIX_BYTES = None  # filled from the spec


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def matrix_bytes(rows, cols):
    return rows * cols // 2 + rows * cols // 32


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=("decode", "batched", "prefill", "latent", "step", "cache", "stack"), default="decode")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--slots", type=int, default=224, help="cache: HBM expert slots")
    ap.add_argument("--layers", type=int, default=8, help="stack: resident layers")
    ap.add_argument("--tokens", type=int, default=1, help="stack, latent, cache: tokens per step")
    ap.add_argument("--routing", choices=("normal", "zipf"), default=None,
                    help="cache: routing of the token pool (default normal)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the layer is measured "
                          "on one MI355X (expert-parallel sharding is a design note, not a "
                          "measured path)", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp4_routed_expert_sigmoid_amd as k3
    import synth
    import synth.device as sd

    dev = "cuda:0"
    torch.cuda.set_device(0)
    T, routing, pool = {"decode": (1, "normal", 64), "batched": (64, "normal", 8),
                        "prefill": (2048, "zipf", 2), "latent": (args.tokens, "normal", 64 if args.tokens == 1 else 8),
                        "step": (1, "normal", 64), "cache": (args.tokens, "normal", 256 if args.tokens == 1 else 32),
                        "stack": (args.tokens, "normal", 8)}[args.workload]
    nl = args.layers if args.workload == "stack" else 1
    if args.workload == "cache" and args.routing:
        routing = args.routing
    if args.workload == "latent":
        spec = synth.pages_latent_spec(seed=0, routing=routing)
    else:
        spec = synth.full_spec(seed=0, routing=routing)
    H, I, E, K, Is = spec.hidden, spec.inter, spec.n_experts, spec.topk, spec.shared_inter
    Lt, EKw = spec.latent, spec.ek   # latent width (0: flat); width the experts run at
    log(f"[bench] building layer: {E} experts x {spec.expert_bytes} B resident")
    tens = sd.layer_tensors(spec, 0, dev)
    layer = sd.make_layer(spec, tens)
    cache = None
    if args.workload == "cache":
        # the routed experts move to pinned host memory; HBM keeps --slots of them
        host = dict(tens)
        for k in ("gate_packed", "gate_scales", "up_packed", "up_scales", "down_packed", "down_scales"):
            h = torch.empty(tens[k].shape, dtype=tens[k].dtype, pin_memory=True)
            h.copy_(tens[k])
            host[k] = h
        torch.cuda.synchronize()
        layer.close()
        del layer
        tens = host
        torch.cuda.empty_cache()
        layer = sd.make_layer(spec, tens)
        cache = k3.Cache(layer, args.slots)
        log(f"[bench] experts in pinned host memory, {args.slots} HBM slots")
    layers = [layer]
    for l in range(1, nl):
        log(f"[bench] building layer {l}")
        layers.append(sd.make_layer(spec, sd.layer_tensors(spec, l, dev)))
    xs_np = [synth.make_x(spec, T, attempt=100 + p) for p in range(pool)]
    xs = [sd.bf16_tensor(x, dev) for x in xs_np]
    ws = layer.workspace(T) if cache is None else cache.workspace(T)
    idxs = [torch.empty((T, K), dtype=torch.int32, device=dev) for _ in range(nl)]
    ws_l = [torch.empty((T, K), dtype=torch.float32, device=dev) for _ in range(nl)]
    idx, w = idxs[0], ws_l[0]
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    if args.workload == "step":
        # residual streams (each step adds the layer's output into its row)
        hs_np = [synth.make_residual(spec, T, attempt=100 + p) for p in range(pool)]
        hs = [torch.from_numpy(h).to(dev) for h in hs_np]
        gamma_np = synth.make_post_norm(spec)
        gamma = torch.from_numpy(gamma_np).to(dev)
    if args.workload == "stack":
        hs_np = [synth.make_residual(spec, T, attempt=100 + p) for p in range(pool)]
        hs = [torch.from_numpy(h).to(dev) for h in hs_np]
        gammas = [torch.from_numpy(synth.make_post_norm(spec, l)).to(dev) for l in range(nl)]
        gamma_np = synth.make_post_norm(spec, 0)

    # calibration read of known size (256 MiB) for hardware byte counters
    cal = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sd.read_probe(cal, sink)
    del cal

    def step(i):
        if args.workload == "stack":
            h = hs[i % pool]
            for l, lay in enumerate(layers):
                lay.step(h, gammas[l], STEP_EPS, idxs[l], ws_l[l], workspace=ws, stream=stream)
            return
        if args.workload == "step":
            layer.step(hs[i % pool], gamma, STEP_EPS, idx, w, workspace=ws, stream=stream)
            return
        x = xs[i % pool]
        if cache is not None:
            layer.route(x, idx, w, workspace=ws, stream=stream)
            cache.forward(x, idx, w, out, workspace=ws, stream=stream)
            return
        layer.route_forward(x, idx, w, out, workspace=ws, stream=stream)

    # distinct experts per pool entry (for the algorithmic byte counts)
    distinct, heavy = [], []
    for p in range(pool):
        step(p)
        torch.cuda.synchronize()
        dl, hl = [], []
        for l in range(nl):   # per layer; a stack's figures are per-layer means
            ids = idxs[l].cpu().numpy().ravel()
            dl.append(len(set(ids.tolist())))
            cnt = np.bincount(ids[(ids >= 0) & (ids < E)], minlength=E)
            hl.append(cnt[cnt > STREAM_MAX_TOKENS])   # experts the tile GEMMs take
        distinct.append(sum(dl) / nl)
        heavy.append(np.concatenate(hl) if nl > 1 else hl[0])
    assert layer.error_count() == 0

    if cache is not None:
        # fill the arena and reach the steady state before timing
        for i in range(max(args.warmup, 4 * E // K)):
            step(i)
        torch.cuda.synchronize()
        c0 = cache.stats()
    else:
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    log(f"[bench] timed {args.steps} steps: {ms:.4f} ms/step")
    if cache is not None:
        c1 = cache.stats()
        cd = {k: c1[k] - c0[k] for k in c1}

    # per-step spread: an event pair around every step (same steps), so the
    # median and the 10th / 90th percentiles of the step time can be reported
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    step_us = np.sort(np.array([a.elapsed_time(b) * 1e3 for a, b in evs]))
    pct = {q: float(np.percentile(step_us, q)) for q in (10, 50, 90)}
    log(f"[bench] step us p10 {pct[10]:.2f} p50 {pct[50]:.2f} p90 {pct[90]:.2f}")

    # second pass with per-stage events (same steps): an event pair around
    # each stage's launches on the launch stream; a stage's time is summed
    # over its launches in a step (a batch of 2-4 tokens runs the one-token
    # kernels once per token) and averaged over the steps
    layer.profile(True)
    layer.profile_read(stream)
    for i in range(args.steps):
        step(i)
    stages = layer.profile_read(stream)
    layer.profile(False)
    stage_us = {k: v[0] * 1e3 / args.steps for k, v in stages.items() if v[1]}
    launches = {k: v[1] / args.steps for k, v in stages.items() if v[1]}
    log(f"[bench] stage us/step: " + ", ".join(f"{k} {v:.2f}" for k, v in stage_us.items()))

    # algorithmic bytes, averaged over the rotation actually timed
    nd = sum(distinct[i % pool] for i in range(args.steps)) / args.steps
    gu = matrix_bytes(I, EKw)
    dn = matrix_bytes(EKw, I)
    expert_b = 2 * gu + dn
    routed_bytes = nd * expert_b
    router_bytes = E * H * 2
    shared_bytes = 3 * Is * H * 2
    proj_bytes = 2 * Lt * H * 2 + Lt * 4   # latent down- and up-projection, norm weights
    # per stage: weights read once, token side read, activations written/read
    # (4 B per element: fp32, or bf16 hi + lo), expert outputs staged in fp32
    x_read = T * H * 2 + (T * Lt * 4 if Lt else 0)   # the bf16 tokens (+ the latent's hi/lo planes)
    act_b = T * K * I * 4 + T * Is * 4
    # the fused one-token kernels (a flat layer, 1..8 tokens, no combine
    # stage), once per token: router | shared gate/up + (at one token the
    # top-k) + routed gate/up | shared down + routed down + router-order sum;
    # each token's pass reads its own experts and the shared expert again
    fused = "combine" not in stage_us and not Lt and T <= 8 and cache is None
    # the older single-token kernels once per token, then one combine
    per_token = not fused and not Lt and T <= 4 and cache is None
    if fused:
        terms = K * 3 * I + K * 3 * (I // 32)   # the activations as three e4m3 terms and their scales
        scores = E * 8 if T == 1 else 0          # the fused top-k reads the scores
        epi = H * 4 * (2 if args.workload in ("step", "stack") else 1)
        stage_bytes = {
            "router": router_bytes + T * H * 2 + T * E * 8,
            "gateup": T * (K * 2 * gu + 2 * Is * H * 2 + H * 2 + terms + Is * 4 + K * 8) + scores,
            "down": T * (K * dn + Is * H * 2 + terms + Is * 4 + K * 8 + epi),
        }
    elif per_token:
        # the older single-token kernels, one pass per token
        stage_bytes = {
            "gateup": T * (K * 2 * gu + 2 * Is * H * 2 + H * 2 + K * I * 4 + Is * 4),
            "down": T * (K * dn + Is * H * 2 + K * I * 4 + Is * 4 + (K + 1) * H * 4),
        }
    else:
        shared_in_gateup = "shared_gateup" not in stage_us  # no separate shared gate/up launch
        stage_bytes = {
            "gateup": nd * 2 * gu + (2 * Is * H * 2 if shared_in_gateup else 0) + x_read + act_b,
            "down": nd * dn + Is * H * 2 + act_b + T * (K + 1) * EKw * 4 + (T * H * 4 if Lt else 0),
        }
    if args.workload in ("step", "stack"):
        if T == 1 and fused:   # the norm runs in the router's launch
            stage_bytes["router"] += T * H * 4 + H * 4 + T * H * 2
        else:
            stage_bytes["prenorm"] = T * H * 4 + H * 4 + T * H * 2
    if cache is not None:
        stage_bytes = {"cache_fill": cd["bytes_read"] / max(1, cd["steps"])}
    if Lt:
        stage_bytes["latent_in"] = Lt * H * 2 + T * H * 2 + T * Lt * 4
        stage_bytes["latent_out"] = H * Lt * 2 + Lt * 4 + T * Lt * 12 + T * H * 8
    one_tok = {"gateup": "k_gateup_dec", "down": "k_down_dec"}   # the older per-token loop's kernels
    fused_k = {"router": "k_router", "gateup": "k_dec_gateup", "down": "k_dec_down"}
    stream_k = {"gateup": "k_gu_stream", "down": "k_dn_stream"}
    step_k = (dict(fused_k, router="k_prenorm_router") if fused and T == 1
              else dict(fused_k, prenorm="k_prenorm") if fused
              else dict(one_tok, prenorm="k_prenorm") if per_token
              else dict(stream_k, prenorm="k_prenorm"))
    kernels = {"decode": fused_k if fused else one_tok,
               "batched": fused_k if fused else one_tok if per_token else stream_k,
               "prefill": {"gateup": "k_gu_gemm + k_gu_stream", "down": "k_dn_gemm + k_dn_stream"},
               "latent": ({"gateup": "k_gateup_dec", "down": "k_down_dec", "latent_in": "k_gv_down",
                           "latent_out": "k_gv_up"} if T == 1 else
                          {"gateup": "k_gu_stream", "down": "k_dn_stream", "latent_in": "k_proj",
                           "latent_out": "k_proj + k_rms_split"}),
               "step": step_k,
               "cache": {"cache_fill": "k_cache_fill"},
               "stack": step_k}[args.workload]
    # the hot experts' tile GEMMs: algorithmic flops (2 per multiply-add,
    # gate and up, per assignment) and issued flops (whole token tiles). A flat
    # layer's shared gate/up tiles run in the same launch once the shared
    # expert leaves the streaming kernels (T > 128): their flops count too.
    # The routed down tiles multiply three e4m3 terms of the activation (a
    # latent layer's: bf16 hi and lo).
    tile_tok_gu = 64 if Lt else 128
    sh_in_tiles = not Lt and Is > 0 and T > 128
    dn_terms = 2 if Lt else 3
    mf = {"alg_gu": 0.0, "iss_gu": 0.0, "alg_dn": 0.0, "iss_dn": 0.0}
    for i in range(args.steps):
        c = heavy[i % pool]
        mf["alg_gu"] += c.sum() * 2 * 2 * I * EKw
        mf["iss_gu"] += (np.ceil(c / tile_tok_gu) * tile_tok_gu).sum() * 2 * 2 * I * EKw * (2 if Lt else 1)
        if sh_in_tiles and c.size:
            mf["alg_gu"] += T * 2 * 2 * Is * H
            mf["iss_gu"] += np.ceil(T / 128) * 128 * 2 * 2 * Is * H
        mf["alg_dn"] += c.sum() * 2 * EKw * I
        mf["iss_dn"] += (np.ceil(c / 64) * 64).sum() * 2 * EKw * I * dn_terms
    mf = {k: v / args.steps / nl for k, v in mf.items()}
    dom = max(stage_bytes, key=lambda s: stage_us.get(s, 0.0))
    dom_us = stage_us.get(dom, 0.0)
    achieved = stage_bytes[dom] / (dom_us * 1e-6) / 1e9 if dom_us > 0 else 0.0
    peak = HBM_PEAK_GBPS if cache is None else HOST_LINK_PEAK_GBPS
    prof_rec = profiled_kernel(kernels[dom]) if T == 1 else None   # the record is of one-token dispatches
    traffic = prof_rec.get("hbm_bytes") if prof_rec else None
    value = nl * routed_bytes / (ms * 1e-3) / 1e9
    layer_bytes = routed_bytes + router_bytes + shared_bytes + proj_bytes + T * H * 2 + T * H * 4
    if args.workload == "stack":
        layer_bytes += T * H * 16 + H * 4   # the stream: norm read, add read + write; the gain
    if args.workload == "step":
        layer_bytes += T * H * 8 + H * 4   # the stream read twice (norm, add) and the gain
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: T={T} tokens/step, "
                        + (f"{nl} resident layers, each a decoder-layer step (pre-MoE RMSNorm, its own "
                           f"router, residual add; k3moe_step), " if args.workload == "stack" else "")
                        + f"hidden {H}, {E} experts top-{K}, "
                        + ("pre-MoE RMSNorm of an fp32 residual stream into bf16 tokens and the "
                           "residual add (k3moe_step), " if args.workload == "step" else "")
                        + (f"experts in a {Lt} latent (bf16 down/up projections, RMSNorm of the "
                           f"aggregate), " if Lt else "")
                        + f"expert inter {I} (MXFP4), bf16 shared expert inter {Is}, sigmoid "
                        f"router + bias N(0,0.01), {routing} routing",
            "tokens_per_step": T,
            "distinct_experts_per_step": round(nd, 2),
        },
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "step_us_p10_p50_p90": [round(pct[10], 2), round(pct[50], 2), round(pct[90], 2)],
        "layer_GBps": round(nl * layer_bytes / (ms * 1e-3) / 1e9, 2),
        "layers_per_step": nl,
        "tokens_per_s_per_layer": round(T * nl / (ms * 1e-3), 1),
        "routed_frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "stage_us_per_step": {k: round(v, 3) for k, v in stage_us.items()},
        "roofline": {
            "kernel": kernels[dom],
            "bound": "hbm" if cache is None else "host link (PCIe 5.0 x16)",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "GB/s",
            "frac": round(achieved / peak, 4),
            "bytes_per_step": round(stage_bytes[dom]),
            "us_per_step": round(dom_us, 3),
            "launches_per_step": round(launches.get(dom, 0.0), 3),
            "timing": "HIP events around the stage's launches on the launch stream, summed per step",
            "traffic": traffic,
        },
    }
    if prof_rec and prof_rec.get("rocprof_avg_us") and launches.get(dom, 0.0) == 1.0:
        # the same kernel's average duration from the committed rocprofv3 kernel trace
        # (profiles/layer_decode_T1_kernel_stats.md), for the same source file
        pu = prof_rec["rocprof_avg_us"]
        result["roofline"]["rocprof"] = {"avg_us": pu,
                                         "achieved": round(stage_bytes[dom] / (pu * 1e-6) / 1e9, 2),
                                         "frac": round(stage_bytes[dom] / (pu * 1e-6) / 1e9 / peak, 4)}

    if mf["alg_gu"] > 0 and stage_us.get("gateup_tiles", 0) > 0:
        tu, td = stage_us["gateup_tiles"] * 1e-6, max(stage_us.get("down_tiles", 0), 1e-9) * 1e-6
        result["mfma"] = {
            "kernel": "k_gemm gate/up tiles (experts with > 16 assignments"
                      + (", and the shared expert's)" if sh_in_tiles else ")"),
            "alg_TFLOPs": round(mf["alg_gu"] / tu / 1e12, 2),
            "issued_TFLOPs": round(mf["iss_gu"] / tu / 1e12, 2),
            "alg_frac_of_mxfp4_peak": round(mf["alg_gu"] / tu / 1e12 / MXFP4_PEAK_TFLOPS, 4),
            "issued_frac_of_bf16_peak": round(mf["iss_gu"] / tu / 1e12 / BF16_PEAK_TFLOPS, 4),
            "down_alg_TFLOPs": round(mf["alg_dn"] / td / 1e12, 2),
            ("down_issued_frac_of_bf16_peak" if Lt else "down_issued_frac_of_fp8_peak"):
                round(mf["iss_dn"] / td / 1e12 / (BF16_PEAK_TFLOPS if Lt else FP8_PEAK_TFLOPS), 4),
            "tile_us": [round(stage_us["gateup_tiles"], 2), round(stage_us.get("down_tiles", 0.0), 2)],
        }
        if args.workload == "prefill":   # the dominant kernel is the hot experts' gate/up tiles
            a = mf["alg_gu"] / tu / 1e12
            result["roofline"] = {"kernel": "k_gemm<0> (gate/up tiles)", "bound": "mfma",
                                  "achieved": round(a, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(a / BF16_PEAK_TFLOPS, 4),
                                  "flops_per_launch": round(mf["alg_gu"]), "traffic": None}
    if cache is not None:
        result["config"]["workload"] += f", experts in pinned host memory, {args.slots} HBM slots"
        result["cache"] = {
            "slots": args.slots,
            "requests_per_step": round(cd["requests"] / cd["steps"], 3),
            "resident_hit_rate": round(cd["resident_hits"] / max(1, cd["requests"]), 4),
            "retention": round(1 - cd["evictions"] / max(1, cd["requests"]), 4),
            "host_bytes_per_step": round(cd["bytes_read"] / cd["steps"]),
            "dropped": cd["dropped"],
            "slots_over_experts": round(args.slots / E, 4),
        }
    if not args.no_cpu_baseline:
        if args.workload in ("step", "stack"):
            result["cpu_baseline"] = cpu_baseline(spec, hs_np, T, args.cpu_seconds, expert_b,
                                                  gamma=gamma_np)
        else:
            result["cpu_baseline"] = cpu_baseline(spec, xs_np, T, args.cpu_seconds, expert_b)
    print(json.dumps(result), flush=True)


def profiled_kernel(kernel):
    """The committed rocprofv3 record of `kernel` (profiles/decode_T1_pmc_traffic.json):
    HBM bytes per dispatch from the FETCH_SIZE and WRITE_SIZE counter runs
    (each scaled by what the counter reads for a copy of known size) and the
    kernel's average duration in the kernel trace, or None when no such
    record exists or the kernel's source file has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode_T1_pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel)
    if k is None or "source" not in k or "source_sha256" not in k:
        return None
    src = os.path.join(ROOT, k["source"])
    if not os.path.exists(src):
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != k["source_sha256"]:
            return None
    return k


def cpu_baseline(spec, xs_np, T, budget_s, expert_b, gamma=None, distinct=16):
    """The fp64 oracle (route + forward) on this host, on whole tokens of the
    same workload until about budget_s seconds of oracle time have passed:
    the first `distinct` tokens of the input pool, over and over. Their
    experts' bytes are generated on the host once, outside the timed region.
    With gamma, xs_np holds residual streams and the oracle's pre-MoE norm
    makes the tokens (timed)."""
    import itertools

    import numpy as np

    import oracle
    import synth

    Wr = synth.make_router(spec)
    bias = synth.make_bias(spec)
    shared = synth.make_shared(spec)
    lat = synth.make_latent(spec)
    cand = [(p, t) for t in range(T) for p in range(len(xs_np))][:distinct]
    # the experts of the sample's tokens, generated once (untimed)
    first = []
    for p, t in cand:
        x = xs_np[p][t:t + 1]
        if gamma is not None:
            x = oracle.prenorm_bf16(x, gamma, STEP_EPS)
        first.append(oracle.route(x, Wr, bias, spec.topk)[0])
    used = sorted({int(e) for idx in first for e in idx.ravel()})
    h = synth.expert_host(spec, used)
    es = oracle.ExpertSet(used, spec.n_experts, h["gate_packed"], h["gate_scales"],
                          h["up_packed"], h["up_scales"], h["down_packed"], h["down_scales"])
    del h
    spent = 0.0
    next_log = 2.0
    tokens = 0
    routed = 0
    for p, t in itertools.cycle(cand):
        x = xs_np[p][t:t + 1]
        t0 = time.perf_counter()
        if gamma is not None:
            x = oracle.prenorm_bf16(x, gamma, STEP_EPS)
        idx, w = oracle.route(x, Wr, bias, spec.topk)
        if spec.latent:
            wd, wu, g_lat = lat
            oracle.forward_latent(x, idx, w, es, spec.hidden, spec.latent, spec.inter, wd, wu,
                                  norm=bool(spec.latent_norm), gamma=g_lat, eps=spec.rms_eps,
                                  shared=shared, act_kind=spec.act, b1=spec.situ_b1, b2=spec.situ_b2,
                                  want_denom=False)
        else:
            oracle.forward(x, idx, w, es, spec.hidden, spec.inter, shared=shared,
                           act_kind=spec.act, b1=spec.situ_b1, b2=spec.situ_b2, want_denom=False)
        spent += time.perf_counter() - t0
        tokens += 1
        routed += len(set(idx.ravel().tolist())) * expert_b
        if spent >= next_log:
            log(f"[bench] cpu baseline: {tokens} tokens, {spent:.1f} s")
            next_log += 2.0
        if spent >= budget_s:
            break
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(routed / spent / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(tokens / spent, 4),
        "cores": oracle.threads(),
        "cpu_model": model,
        "nproc": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{tokens} whole tokens (route + {spec.topk} experts + shared expert), one per oracle "
                  f"call, cycling over the first {len(cand)} tokens of this workload's inputs; "
                  f"{spent:.1f} s of oracle time",
    }


if __name__ == "__main__":
    main()
