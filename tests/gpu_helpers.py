"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import numpy as np

import oracle
import synth

# Bound on |ch_gpu - ch_oracle| for one expert. The oracle's logit is the
# fp64 sum of the exact bf16 products; the one-wave GPU router's is another
# fp64 sum of them (one fp32 ulp apart at most), the batch router's an fp64
# sum of fp32 sums of 32 products (see LOGIT_REL; the tests check this bound
# on its logits directly). A logit difference d
# moves the fp32 score by at most d/4 + one rounding (2^-24) and the
# selection score by one more rounding of a value below 2. Gaps above twice
# this bound cannot reorder the selection.
CH_DELTA = 2.0 ** -20

# Max relative error of an output element, |gpu - oracle| / D, where D is the
# oracle's magnitude sum sum_j |w_j| sum_n |W2[o][n] a_j[n]| + shared terms
# (a latent layer: the same magnitude carried through the norm and the
# up-projection).
REL_TOL = 1e-4

# Logits. The batch router sums each run of 32 exact products in fp32 (at
# most 31 roundings, each at most 2^-23 of the running sum even if the MFMA
# truncated) before adding the runs in fp64, so its logit is within
# 2^-18 sum_k |x_k w_k| of the exact sum; the fp32 rounding of the logit adds
# at most one ulp. That bound is the check on the logits themselves; route
# parity rests on the selection scores, which check_logits also recomputes
# from the GPU's fp32 logits (the router's formula: fp64 sigmoid rounded to
# fp32, plus the fp32 bias) and holds within CH_DELTA of the oracle's.
LOGIT_REL = 2.0 ** -18


def logit_magnitudes(x, Wr, rows=None):
    """sum_k |x_k w_k| for every (token, expert) of the listed rows (fp64)."""
    X = np.abs(synth.bf16_to_f32(x if rows is None else x[rows]).astype(np.float64))
    return X @ np.abs(synth.bf16_to_f32(Wr).astype(np.float64)).T


def check_logits(lg_gpu, logits_ref, ch_ref, bias, mag):
    """Asserts the GPU's fp32 logits within LOGIT_REL * mag + one ulp of the
    oracle's, and the selection scores they give within CH_DELTA of the
    oracle's. Returns (largest |difference| beyond one ulp over mag, largest
    selection-score difference) for the log."""
    ref32 = logits_ref.astype(np.float32)
    d = np.abs(lg_gpu.astype(np.float64) - ref32.astype(np.float64))
    excess = np.maximum(d - np.spacing(np.abs(ref32)).astype(np.float64), 0.0) / np.maximum(mag, 1e-300)
    assert float(excess.max()) <= LOGIT_REL, (float(d.max()), float(excess.max()))
    s = (1.0 / (1.0 + np.exp(-lg_gpu.astype(np.float64)))).astype(np.float32)
    ch = s + (bias.astype(np.float32) if bias is not None else np.float32(0.0))
    dch = float(np.abs(ch.astype(np.float64) - ch_ref.astype(np.float64)).max())
    assert dch <= CH_DELTA, dch
    return float(excess.max()), dch


def route_certificate(ch, topk, delta=CH_DELTA):
    """Per token: True when every adjacent gap among the top k+1 selection
    scores (oracle fp32 values, order ch desc / expert asc) exceeds 2*delta."""
    T, E = ch.shape
    ok = np.zeros(T, bool)
    for t in range(T):
        order = np.lexsort((np.arange(E), -ch[t].astype(np.float64)))[: min(E, topk + 1)]
        v = ch[t, order].astype(np.float64)
        ok[t] = bool(np.all(np.abs(np.diff(v)) > 2 * delta)) if v.size > 1 else True
    return ok


# Routing weights, relative. A weight is a score over the sum of the selected
# scores (times a constant): a logit difference d moves a score by at most
# d (1 - s) relative plus one fp32 rounding. The batch router's logits stay
# within a few 2^-21 of the oracle's on the workloads here (largest seen
# 1.9e-6, at |logit| in [4, 8)), so its weights agree within 2^-17; the
# one-wave router (T <= 4) sums the same products as the oracle in fp64: its
# scores are the oracle's but for a rare one-ulp logit, and its weights agree
# within a few ulps.
W_RTOL_BATCH = 2.0 ** -17
W_RTOL_WAVE = 4e-7


def check_route(idx_gpu, w_gpu, idx_ref, w_ref, ch_ref, topk, delta=CH_DELTA, w_rtol=W_RTOL_BATCH):
    """Exact indices on certified tokens; on the others the GPU's choice must
    be a valid top-k under +-delta perturbations of the scores. Weights within
    w_rtol of the oracle's. Returns the number of certified tokens."""
    cert = route_certificate(ch_ref, topk, delta)
    for t in range(idx_ref.shape[0]):
        if cert[t]:
            assert np.array_equal(idx_gpu[t], idx_ref[t]), (t, idx_gpu[t], idx_ref[t])
            np.testing.assert_allclose(w_gpu[t], w_ref[t], rtol=w_rtol, atol=0)
        else:
            g = ch_ref[t, idx_gpu[t]].astype(np.float64)
            r = ch_ref[t, idx_ref[t]].astype(np.float64)
            assert len(set(idx_gpu[t].tolist())) == topk
            assert np.all(np.abs(g - r) <= 2 * delta), (t, g, r)
    return int(cert.sum())


def rel_err(out_gpu, out_ref, denom):
    err = np.abs(out_gpu.astype(np.float64) - out_ref)
    d = np.where(denom > 0, denom, 1.0)
    assert np.all(err[denom == 0] <= 1e-30)
    return float((err / d).max())


# attempt numbers of redrawn tokens: row t, redraw a -> _REDRAW + t * 64 + a
_REDRAW = 1 << 24
_REDRAW_MAX = 64


def certify_rows(spec, x, Wr, bias, rows=None, layer=0):
    """Redraw, in place, every listed token of x (bf16 patterns [T][H]) whose
    oracle route is not certified: row t takes the single token
    synth.make_x(spec, 1, layer, attempt=_REDRAW + 64 t + a) for the next a
    until its route is. Returns the oracle's (idx, w, logits, ch) of the
    listed rows (all rows by default), every one certified, so the GPU's ids
    must equal the oracle's exactly on them."""
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    kw = dict(renorm=spec.renorm, routed_scale=spec.routed_scale, want_detail=True)
    res = list(oracle.route(x[rows], Wr, bias, spec.topk, **kw))
    for a in range(_REDRAW_MAX):
        bad = np.nonzero(~route_certificate(res[3], spec.topk))[0]
        if bad.size == 0:
            return tuple(res)
        for i in bad:
            t = int(rows[i])
            x[t] = synth.make_x(spec, 1, layer=layer, attempt=_REDRAW + t * _REDRAW_MAX + a)[0]
        for arr, new in zip(res, oracle.route(x[rows[bad]], Wr, bias, spec.topk, **kw)):
            arr[bad] = new
    raise AssertionError("a token stayed uncertified")


def tile_edge_tokens(idx, n_experts, smax, tile_sizes, experts=None):
    """Tokens on the edges of the grouped-GEMM tiles. The permutation lists an
    expert's assignments in token order; an expert with more than smax of
    them runs on tiles of each listed size. For each such expert (or each
    listed one): the tokens in the first and last row of its first tile, the
    first row of its second tile, and the first and last row of its last
    (possibly partial) tile."""
    out = set()
    for e in (range(n_experts) if experts is None else experts):
        toks = np.nonzero((idx == e).any(1))[0]
        n = toks.size
        if n <= smax:
            continue
        for ts in tile_sizes:
            rows = {0, min(ts, n) - 1, ts * ((n - 1) // ts), n - 1}
            if n > ts:
                rows.add(ts)
            out.update(int(toks[r]) for r in rows)
    return sorted(out)


_SHARED = {}


def _shared(spec, layer):
    """synth.make_shared, kept for the last few (spec, layer) pairs."""
    key = (repr(spec), layer)
    if key not in _SHARED:
        if len(_SHARED) >= 4:
            _SHARED.pop(next(iter(_SHARED)))
        _SHARED[key] = synth.make_shared(spec, layer)
    return _SHARED[key]


def oracle_forward(spec, x, idx, w, layer=0, tokens=None, chunk=48):
    """Oracle output/denominators for the listed tokens (all by default), in
    chunks of tokens (the host copies of one chunk's experts at a time)."""
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens)
    if tokens.size > chunk:
        parts = [oracle_forward(spec, x, idx, w, layer, tokens[i:i + chunk], chunk)
                 for i in range(0, tokens.size, chunk)]
        return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
                sum(p[2] for p in parts))
    xs, ids, ws = x[tokens], idx[tokens], w[tokens]
    used = sorted({int(e) for e in ids.ravel() if 0 <= e < spec.n_experts})
    h = synth.expert_host(spec, used, layer)
    es = oracle.ExpertSet(used, spec.n_experts, h["gate_packed"], h["gate_scales"],
                          h["up_packed"], h["up_scales"], h["down_packed"], h["down_scales"])
    shared = _shared(spec, layer)
    if spec.latent:
        wd, wu, gamma = synth.make_latent(spec, layer)
        return oracle.forward_latent(xs, ids, ws, es, spec.hidden, spec.latent, spec.inter, wd, wu,
                                     norm=bool(spec.latent_norm), gamma=gamma, eps=spec.rms_eps,
                                     shared=shared, act_kind=spec.act, b1=spec.situ_b1, b2=spec.situ_b2)
    out, denom, drops = oracle.forward(xs, ids, ws, es, spec.hidden, spec.inter, shared=shared,
                                       act_kind=spec.act, b1=spec.situ_b1, b2=spec.situ_b2)
    return out, denom, drops


def bf16_rne_np(v):
    """bf16 bits of fp32 values by the definition (nearer neighbour, ties to
    the even one), vectorised."""
    v = np.asarray(v, np.float32)
    toward = (v.view(np.uint32) >> 16).astype(np.uint32)
    away = toward + 1
    f = lambda b: (b << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    dt = np.abs(v.astype(np.float64) - f(toward))
    da = np.abs(f(away) - v.astype(np.float64))
    pick_away = (da < dt) | ((da == dt) & ((toward & 1) == 1))
    return np.where(pick_away, away, toward).astype(np.uint16)
