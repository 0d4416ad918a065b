"""GPU-vs-oracle parity protocol shared by the GPU tests.

Both sides get the same seeded weights and prompts.  At every decode step the
oracle runs first; its token is fed to both sides (teacher forcing), and where
an exit decision of the oracle lies within 1e-3 of gamma the GPU is forced to
the oracle's exit layer for that sequence.

bf16 activations make exact agreement of near-ties impossible to guarantee:
the two sides accumulate in different precisions (float64 vs float32), so a
value close to a bf16 rounding midpoint rounds differently now and then, and
one flipped SwiGLU output moves the residual by ~1e-3 relative.  The bands
below are therefore the stated ones widened by the discrepancy measured in the
same step (which itself must stay within the tolerances):
  * exit layers must match exactly.  A differing exit layer is accepted only
    when the oracle's value at the first differing decision lies within the
    bound below of the threshold (so the measured error of the head's input
    can carry it across) and the GPU's value is within that bound of the
    oracle's; that step is then rolled back (ee_kv_cache_rollback) and re-run
    with the oracle's exit layer forced for that sequence (teacher forcing),
    and compared again.  Such exits are counted ("widened exits");
  * tokens must match exactly where the oracle's top-2 logit gap exceeds
    max(1e-2, 2 * max|logit_gpu - logit_oracle|) of that sequence;
  * KV slot occupancy must match exactly,
  * logits, hidden states (after every layer) and K/V must agree within a max
    relative error of 2e-2 (max |gpu - oracle| / max |oracle| per tensor),
  * exit-head probabilities must agree to what the measured error of the
    head's input implies (head_lnp_bound): the GPU's hidden state after the
    layer and the oracle's, each rounded to bf16, are pushed through T (with
    the float32 summation error of the GPU's z = T a, which can move z_j only
    between bf16(y_j - eps_j) and bf16(y_j + eps_j)) and through E (with the
    float32 error of each logit's sum); p = 1 / sum_v exp(l_v - max l), so
    moving every logit by at most d moves ln p by at most 2 d; 1e-4 covers
    the fast exponential and the float32 merge of the per-workgroup sums;
  * with the state-transition-similarity criterion, the similarity after
    layer l must agree to what the hidden states' agreement implies: moving
    a by da changes cos(a, b) by at most 2 |da| / |a|, so
    |s_gpu - s_oracle| <= 2 (r_{l-1} + r_l) + 1e-6 with r the norm-relative
    error of the GPU's hidden state before and after the layer (the same
    bound decides whether a differing exit is a near tie).
"""
from __future__ import annotations

import sys
import time

import numpy as np

import synth
from oracle import model as om
from oracle.numerics import from_bf16_bits

TOL = 2e-2
GAP_BAND = 1e-2
P_BAND = 1e-3
# sampled decoding: a draw's perturbed top-2 gap (score units: logit / tau plus
# Gumbel noise, float32 on the GPU) and the acceptance test's relative margin
# |u p_draft - p_final| / max(p_draft, p_final) below which the decision is a
# near tie (the logit error is added to the gap band by the caller)
SAMPLE_BAND = 2e-3
ACCEPT_BAND = 1e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def maxrel(a, r):
    a = np.asarray(a, np.float64)
    r = np.asarray(r, np.float64)
    den = np.abs(r).max()
    if den == 0:
        return float(np.abs(a).max())
    return float(np.abs(a - r).max() / den)


class Result:
    def __init__(self):
        self.compared_tokens = 0
        self.tie_tokens = 0
        self.forced_rows = 0
        self.widened_exits = 0
        self.widened_tokens = 0
        self.exits = []
        self.worst = {}
        self.sample_outcomes = []   # sampled decoding: "none" / "accepted" / "rejected" per compared token

    def note(self, key, v):
        self.worst[key] = max(self.worst.get(key, 0.0), v)


U32 = 2.0 ** -24
LNP_SLACK = 1e-4
LAMBDA = 8.0   # standard deviations of the float32 summation error model below


def _sum_err(M, x, chunk=8192, cache=None):
    """Float32 summation error allowance of each row sum of M * x (M float64
    [n, d]): LAMBDA standard deviations of recursive summation with
    independent rounding errors (each |delta| <= 2^-24, standard deviation
    2^-24 / sqrt(3)) on partial sums that grow like a random walk, i.e.
    LAMBDA * 2^-24 * sqrt(d / 6) * ||M_row * x||_2.  Worst-case bounds
    ((d + 1) 2^-24 sum |M_row x|) exceed a bf16 unit at d = 4096 and would
    put an interval on every output; the GPU's blocked sums (per lane, then
    across lanes) err less than recursive summation.  ``cache`` keeps M**2."""
    d = M.shape[1]
    x2 = np.asarray(x, np.float64) ** 2
    out = np.empty(M.shape[0])
    for i in range(0, M.shape[0], chunk):
        key = ("sq", i)
        if cache is not None and key in cache:
            m2 = cache[key]
        else:
            m2 = (M[i:i + chunk] ** 2).astype(np.float32)
            if cache is not None:
                cache[key] = m2
        out[i:i + chunk] = m2.astype(np.float64) @ x2 if m2.shape[0] <= 512 else m2 @ x2.astype(np.float32)
    return LAMBDA * U32 * np.sqrt(d / 6.0) * np.sqrt(np.maximum(out, 0.0))


def _abs_matvec(M, x, chunk=16384):
    """|M| @ |x| (M float64 [n, d]) over the nonzero entries of x, in row chunks."""
    ax = np.abs(np.asarray(x, np.float64))
    nz = np.nonzero(ax)[0]
    out = np.zeros(M.shape[0])
    if len(nz):
        for i in range(0, M.shape[0], chunk):
            out[i:i + chunk] = np.abs(M[i:i + chunk][:, nz]) @ ax[nz]
    return out


def head_lnp_bound(orc, layer, h_gpu, h_orc):
    """Bound on |ln p_gpu - ln p_oracle| of the exit head of ``layer`` given the
    GPU's and the oracle's hidden states after that layer (float vectors [d]).

    a = bf16(h_gpu), r = bf16(h_orc).  The GPU sums y_j = (T a)_j in float32,
    off by at most eps_j (_sum_err); rounding to bf16 is monotone, so its z_j
    lies in [lo_j, hi_j] = [bf16(y_j - eps_j), bf16(y_j + eps_j)] (one value
    unless y_j is within eps_j of a rounding midpoint), against the oracle's
    z_o = bf16(T r).  With c the midpoints and rad the half-widths, logit v
    differs by at most |E_v (c - z_o)| + sum_j |E_vj| rad_j + eta_v, eta_v the
    float32 summation allowance of the GPU's logit.  p = 1 / sum exp(l - max l)
    moves ln p by at most twice the largest logit change; LNP_SLACK covers
    the fast exponential and the float32 merge of the per-workgroup sums."""
    from oracle.numerics import bf16_round
    T = orc.w(layer, "head_T")
    E = orc.lm_head
    cache = orc.__dict__.setdefault("_parity_cache", {})
    a = bf16_round(np.asarray(h_gpu, np.float64))
    r = bf16_round(np.asarray(h_orc, np.float64))
    y = T @ a
    eps = _sum_err(T, a, cache=cache.setdefault(("T", layer), {}))
    lo, hi = bf16_round(y - eps), bf16_round(y + eps)
    zo = bf16_round(T @ r)
    c, rad = 0.5 * (lo + hi), 0.5 * (hi - lo)
    zmax = np.maximum(np.abs(lo), np.abs(hi))
    dl = np.abs(E @ (c - zo)) + _abs_matvec(E, rad) + _sum_err(E, zmax, cache=cache.setdefault("E", {}))
    return 2.0 * float(dl.max()) + LNP_SLACK


def _normrel(a, r):
    a = np.asarray(a, np.float64)
    r = np.asarray(r, np.float64)
    return float(np.linalg.norm(a - r) / max(np.linalg.norm(r), 1e-30))


def _value_bound(orc, sts, l, hg, ho):
    """Bound on the difference of the criterion's value after layer l (the
    similarity, or ln p of the exit head) from the rows' traced hidden states
    [L+1, d] on both sides."""
    if sts:
        return 2 * (_normrel(hg[l - 1], ho[l - 1]) + _normrel(hg[l], ho[l])) + 1e-6
    return head_lnp_bound(orc, l, hg[l], ho[l])


def run_parity(shape, weights, batch, P, steps, gamma, exit_mode="int4", forced_fn=None,
               prompts=None, max_seq=None, check_kv=True, check_hidden=True, label="", criterion="head",
               check_every=1, exit_rule="sequence", temperature=0.0, seed=0):
    import torch
    from kv_shared_exit_amd import api, _binding as B

    L = shape.n_layers
    S = max_seq or (P + steps + 1)
    mode = B.EE_EXIT_INT4 if exit_mode == "int4" else B.EE_EXIT_BF16
    sts = criterion == "sts"
    assert check_hidden, "the bounds on the criterion's value need the hidden states"
    t0 = time.time()
    dev = api.upload_weights(weights)
    model = api.Model(shape, dev, gamma=gamma, exit_mode=mode, max_batch=batch, max_positions=S,
                      criterion=B.EE_CRIT_STS if sts else B.EE_CRIT_HEAD, check_every=check_every,
                      exit_rule=B.EE_RULE_BATCH_MIN if exit_rule == "batch_min" else B.EE_RULE_SEQUENCE,
                      temperature=temperature, sample_seed=seed)
    sampled = temperature > 0
    bmin = exit_rule == "batch_min"
    cache = api.KVCache(model, batch, S, track=True)
    orc = om.OracleModel(shape, weights, exit_mode=exit_mode)
    ocache = om.KVCache(shape, batch, S)
    if prompts is None:
        prompts = np.random.default_rng(123).integers(0, shape.vocab, (batch, P)).astype(np.int32)
    res = Result()
    stream = torch.cuda.Stream()
    try:
        tg, lg = api.prefill(model, cache, prompts, stream=stream, logits=True)
        to, info = om.prefill(orc, ocache, prompts)
        for b in range(batch):
            e = maxrel(lg[b], info["logits"][b])
            res.note("logits", e)
            assert e <= TOL, f"{label} prefill b={b} logits maxrel {e:.3g}"
            band = max(GAP_BAND, 2 * float(np.abs(lg[b].astype(np.float64) - info["logits"][b]).max()))
            if info["gap"][b] > band:
                assert tg[b] == to[b], f"{label} prefill token b={b}: gpu {tg[b]} oracle {to[b]}"
                res.compared_tokens += 1
            elif info["gap"][b] > GAP_BAND:
                res.widened_tokens += 1
            else:
                res.tie_tokens += 1
        log(f"[{label}] prefill P={P} B={batch} ok ({time.time() - t0:.1f}s)")
        tok_in = to.astype(np.int32)
        gam = np.broadcast_to(np.asarray(gamma, np.float64), (L - 1,))
        for s in range(steps):
            forced = np.zeros(batch, np.int32) if forced_fn is None else np.asarray(forced_fn(s), np.int32)
            to, eo, io = om.decode_step(orc, ocache, tok_in, gamma=gam, forced=forced, trace=check_hidden,
                                        criterion=criterion, check_every=check_every, exit_rule=exit_rule,
                                        temperature=temperature, seed=seed)
            fg = forced.copy()
            for b in range(batch):
                if forced[b] == 0:
                    pe = io["p"][b]
                    ok = np.isfinite(pe)
                    if np.any(np.abs(pe[ok] - gam[ok]) <= P_BAND):
                        fg[b] = eo[b]
                        res.forced_rows += 1
            if bmin and np.any(fg != forced):   # one row's near tie decides the whole batch
                fg = np.where(forced > 0, forced, eo).astype(np.int32)
            for attempt in range(2):
                dbg = {"p": None, "logits": None, "gap": None}
                if check_hidden:
                    dbg["hidden"] = None
                tgpu, egpu = api.decode_step(model, cache, batch, tokens=tok_in, forced=fg, gamma=gam,
                                             stream=stream, debug=dbg)
                bad = np.nonzero(egpu != eo)[0]
                if len(bad) == 0:
                    break
                assert attempt == 0, f"{label} step {s}: exit layers differ under forcing"
                if bmin:   # the batch minimum decided: compare the minima, then force every row
                    l = int(min(egpu[bad].min(), eo[bad].min()))
                    rows = [b for b in range(batch) if forced[b] == 0 and np.isfinite(io["p"][b, l - 1])]
                    bm_g = min(float(dbg["p"][b, l - 1]) for b in rows)
                    bm_o = min(float(io["p"][b, l - 1]) for b in rows)
                    # the minimum moves by at most the largest per-row bound (in ln p for the head)
                    bnd = max(_value_bound(orc, sts, l, dbg["hidden"][b], io["hidden"][b]) for b in rows)
                    if sts:
                        near = abs(bm_o - gam[l - 1]) <= bnd and abs(bm_g - bm_o) <= bnd
                    else:
                        near = (abs(np.log(bm_o) - np.log(gam[l - 1])) <= bnd and
                                abs(np.log(bm_g) - np.log(bm_o)) <= bnd)
                    assert (bm_g - gam[l - 1]) * (bm_o - gam[l - 1]) <= 0 and near, (
                        f"{label} step {s}: batch exit gpu {egpu} oracle {eo} not a near tie "
                        f"(min gpu {bm_g:.6f} oracle {bm_o:.6f} threshold {gam[l - 1]} bound {bnd:.3g})")
                    fg = np.where(forced > 0, forced, eo).astype(np.int32)
                    res.widened_exits += 1
                    cache.rollback(-1, 1)
                    continue
                for b in bad:
                    l = int(min(egpu[b], eo[b]))          # first decision that differs
                    pg, po = float(dbg["p"][b, l - 1]), float(io["p"][b, l - 1])
                    bound = _value_bound(orc, sts, l, dbg["hidden"][b], io["hidden"][b])
                    if sts:
                        near = abs(po - gam[l - 1]) <= bound and abs(pg - po) <= bound
                    else:
                        near = (abs(np.log(po) - np.log(gam[l - 1])) <= bound and
                                abs(np.log(pg) - np.log(po)) <= bound)
                    assert (pg - gam[l - 1]) * (po - gam[l - 1]) <= 0 and near, (
                        f"{label} step {s} b={b}: exit gpu {egpu[b]} oracle {eo[b]} not a near tie "
                        f"(p gpu {pg:.6f} oracle {po:.6f} gamma {gam[l - 1]} bound {bound:.3g})")
                    fg[b] = eo[b]
                    res.widened_exits += 1
                cache.rollback(-1, 1)
            np.testing.assert_array_equal(egpu, eo, err_msg=f"{label} step {s} exit layers")
            for b in range(batch):
                eps = float(np.abs(dbg["logits"][b].astype(np.float64) - io["logits"][b]).max())
                band = max(GAP_BAND, 2 * eps)
                if sampled:
                    # every decision of the draw (perturbed top-2 gaps; the
                    # acceptance test's relative margin) clear of rounding
                    si = io["sample"][b]
                    mg = si["margins"]
                    gaps = [mg[0]] + mg[2:] if si["draft"] is not None else mg
                    safe = min(gaps) > SAMPLE_BAND + 2 * eps / temperature and (
                        si["draft"] is None or mg[1] > ACCEPT_BAND)
                    if safe:
                        assert tgpu[b] == to[b], (f"{label} step {s} b={b}: sampled token gpu {tgpu[b]} oracle "
                                                  f"{to[b]} ({si})")
                        res.compared_tokens += 1
                        res.sample_outcomes.append("none" if si["draft"] is None else
                                                   "accepted" if si["accepted"] else "rejected")
                    else:
                        res.tie_tokens += 1
                elif io["gap"][b] > band:
                    assert tgpu[b] == to[b], (f"{label} step {s} b={b}: token gpu {tgpu[b]} oracle "
                                              f"{to[b]} gap {io['gap'][b]:.3g} band {band:.3g}")
                    res.compared_tokens += 1
                elif io["gap"][b] > GAP_BAND:
                    res.widened_tokens += 1
                else:
                    res.tie_tokens += 1
                e = maxrel(dbg["logits"][b], io["logits"][b])
                res.note("logits", e)
                assert e <= TOL, f"{label} step {s} b={b} logits maxrel {e:.3g}"
                if check_hidden:
                    for l in range(L + 1):
                        e = maxrel(dbg["hidden"][b, l], io["hidden"][b, l])
                        res.note("hidden", e)
                        assert e <= TOL, f"{label} step {s} b={b} hidden after layer {l}: maxrel {e:.3g}"
                pg, po = dbg["p"][b, :L - 1], io["p"][b]
                np.testing.assert_array_equal(np.isnan(pg), np.isnan(po),
                                              err_msg=f"{label} step {s} b={b} heads evaluated")
                ok = np.isfinite(po)
                if ok.any() and sts:
                    for l in np.nonzero(ok)[0] + 1:
                        bound = 2 * (_normrel(dbg["hidden"][b, l - 1], io["hidden"][b, l - 1]) +
                                     _normrel(dbg["hidden"][b, l], io["hidden"][b, l])) + 1e-6
                        e = abs(float(pg[l - 1]) - float(po[l - 1]))
                        res.note("sts_abs", e)
                        res.note("sts_over_bound", e / bound)
                        assert e <= bound, f"{label} step {s} b={b} layer {l}: similarity err {e:.3g} > {bound:.3g}"
                elif ok.any():
                    e = float(np.abs(pg[ok] - po[ok]).max())
                    res.note("p_abs", e)
                    for l in np.nonzero(ok)[0] + 1:
                        bound = head_lnp_bound(orc, int(l), dbg["hidden"][b, l], io["hidden"][b, l])
                        dl = abs(np.log(float(pg[l - 1])) - np.log(float(po[l - 1])))
                        res.note("lnp_abs", dl)
                        res.note("lnp_bound", bound)
                        res.note("lnp_over_bound", dl / bound)
                        assert dl <= bound, (f"{label} step {s} b={b} layer {l}: ln p err {dl:.3g} > "
                                             f"derived bound {bound:.3g}")
            res.exits.append(eo.copy())
            tok_in = to.astype(np.int32)
        log(f"[{label}] {steps} decode steps ok ({time.time() - t0:.1f}s) worst={res.worst} "
            f"tokens compared={res.compared_tokens} ties={res.tie_tokens} widened={res.widened_tokens} "
            f"forced={res.forced_rows} widened exits={res.widened_exits}")
        occ = cache.occupancy()
        n = P + steps
        np.testing.assert_array_equal(occ[:, :batch, :n], ocache.occ[:, :batch, :n].astype(np.uint8))
        assert np.all(occ[:, :batch, n:] == 0)
        if check_kv:
            for l in range(1, L + 1):
                for b in range(batch):
                    k, v = cache.read(l, b, 0, n)
                    kr = ocache.K[l - 1, b, :, :n].transpose(1, 0, 2)
                    vr = ocache.V[l - 1, b, :, :n].transpose(1, 0, 2)
                    ek = maxrel(from_bf16_bits(k), kr)
                    ev = maxrel(from_bf16_bits(v), vr)
                    res.note("kv", max(ek, ev))
                    assert ek <= TOL and ev <= TOL, f"{label} KV layer {l} seq {b}: {ek:.3g} {ev:.3g}"
        log(f"[{label}] KV/occupancy ok ({time.time() - t0:.1f}s) worst={res.worst}")
    finally:
        cache.close()
        model.close()
    return res
