"""Calibration of the exit heads' logit scales (test infrastructure; see the package header).

Random weights give an exit head with a nearly flat softmax (top-1
probability close to 1/V), so no token would ever cross gamma.  The workloads
ask for a seeded exit-layer distribution instead: tiny mean 1.5 of 4 layers,
1B-shape mean 4.81 of 16 (the figure of the River-LLM explainer, section 2.3),
8B-shape mean 16 of 32, 34B-shape mean 30 of 48.  The target used here is a
truncated geometric distribution with a constant per-layer hazard h (the
probability of exiting after layer l given the token is still on the
backbone), solved so that its mean is the workload's mean.

The head of layer l is scaled by alpha_l (T_l is drawn with standard deviation
0.02 * alpha_l, which scales the logits by alpha_l).  For each calibration
sample (a full-depth hidden state after layer l) the top-1 probability
p(alpha) = max softmax(alpha * logits) increases with alpha, so each sample has
a threshold alpha* with p(alpha*) = gamma and exits at layer l iff
alpha_l > alpha*.  alpha_l is the h-quantile of the samples' alpha*, so a
fraction h of them exit.  This is the analogue, for random weights, of CALM's
threshold tuning on a validation set (CALM explainer, section 4.2).

Samples are the hidden states after every layer of full-depth greedy decode
steps (heads off) that follow a prefill of seeded calibration prompts of the
workload's prompt length, so they cover the positions and the kind of inputs
(the model's own greedy tokens) the workload decodes.  Matrix products run in
float32 here (the oracle's float64 path is used for every parity check).  The
unit-scale logits use T drawn at standard deviation 0.02 without bf16
rounding; the realised exit distribution is therefore close to, not exactly,
the target.  Parity unpinned: this only chooses inputs.

Usage: python -m oracle.calibrate <workload> [--steps N] [--batch B]
writes synth/calibration/<workload>.json.
"""
from __future__ import annotations

import argparse
import json
import os
import time

import numpy as np

import synth
from .model import OracleModel, KVCache, prefill, decode_step, state_transition_similarity
from .numerics import bf16_round, from_bf16_bits


def alpha_threshold(logits: np.ndarray, gamma: float, iters: int = 60) -> np.ndarray:
    """Per row, the alpha > 0 at which max softmax(alpha * logits) equals gamma (bisection in log alpha)."""
    d = logits - logits.max(axis=1, keepdims=True)          # <= 0
    lo = np.full(len(d), -12.0)
    hi = np.full(len(d), 12.0)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        a = np.exp(mid)[:, None]
        p = 1.0 / np.exp(a * d).sum(axis=1)
        up = p > gamma                                         # too confident: lower alpha
        hi = np.where(up, mid, hi)
        lo = np.where(up, lo, mid)
    return np.exp(0.5 * (lo + hi))


def _full_depth_states(wl, steps, calib_batch, prompt_len, say, matmul_dtype):
    """Hidden states [Bc, steps, L+1, d] of full-depth greedy decode steps after a
    prefill of seeded calibration prompts, and the weights with only the heads kept."""
    sh = wl.shape
    L = sh.n_layers
    w = synth.make_weights(sh, wl.seed_weights)
    m = OracleModel(sh, w, exit_mode="bf16", cache_f64=True, matmul_dtype=matmul_dtype)
    for l in range(1, L + 1):                     # widen once, then drop the bf16 copies
        for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "attn_norm", "ffn_norm"):
            m.w(l, name)
        keep = {"head_T": w["layers"][l - 1].get("head_T")}
        w["layers"][l - 1] = keep
    say("weights ready")
    cache = KVCache(sh, calib_batch, prompt_len + steps + 1)
    prompts = synth.make_prompts(wl, batch=calib_batch, length=prompt_len, seed=wl.seed_calib)
    tok, _ = prefill(m, cache, prompts)
    say(f"prefill {calib_batch}x{prompt_len}")
    states = []
    for s in range(steps):
        tok, _, info = decode_step(m, cache, tok, gamma=2.0, trace=True, heads=False)
        states.append(info["hidden"])              # [Bc, L+1, d]
        if s % 32 == 0:
            say(f"decode step {s}")
    del m._f64
    return np.stack(states, axis=1), w


def calibrate_sts(wl, steps: int, calib_batch: int = 4, prompt_len: int | None = None, verbose: bool = True,
                  matmul_dtype=np.float32):
    """Per-layer thresholds tau_l of the state-transition-similarity criterion
    (River-LLM explainer, section 5.2) for workload ``wl``: the row exits after
    layer l iff its similarity > tau_l, so tau_l is the (1 - h) quantile of the
    similarities after layer l of full-depth decode states, and a fraction h
    of them exits (the truncated-geometric hazard of the workload's mean exit
    layer, as for the exit heads).  Parity unpinned: this only chooses inputs."""
    sh = wl.shape
    L = sh.n_layers
    h = synth.geometric_hazard(wl.mean_exit, L)
    P0 = wl.prompt_len if prompt_len is None else prompt_len
    t0 = time.time()

    def say(msg):
        if verbose:
            print(f"[calibrate-sts {wl.name}] {msg} ({time.time() - t0:.0f}s)", flush=True)

    hid, _ = _full_depth_states(wl, steps, calib_batch, P0, say, matmul_dtype)
    # batch-minimum rule: the batch of wl.batch sequences leaves when its
    # smallest similarity > tau; with independent sequences that happens with
    # probability P(s > tau)^B, so the batch hazard is h when each sequence
    # exceeds tau with probability h^(1/B)
    hb = h ** (1.0 / wl.batch)
    taus, taus_b = [], []
    for l in range(1, L):
        sts = state_transition_similarity(hid[:, :, l - 1].reshape(-1, sh.d_model),
                                          hid[:, :, l].reshape(-1, sh.d_model))
        t = float(np.quantile(sts, 1.0 - h))
        tb = float(np.quantile(sts, 1.0 - hb))
        taus.append(t)
        taus_b.append(tb)
        say(f"layer {l}: tau={t:.6f} batch-min tau={tb:.6f} (similarity {sts.min():.4f}..{sts.max():.4f})")
    return {"workload": wl.name, "criterion": "sts", "mean_exit": wl.mean_exit, "hazard": h,
            "samples_per_layer": int(hid.shape[0] * hid.shape[1]),
            "source": f"full-depth greedy decode, {calib_batch} prompts of {P0} tokens, {steps} steps",
            "tau": taus, "batch": wl.batch, "tau_batch_min": taus_b}


def calibrate(wl, steps: int | None = None, calib_batch: int = 4, verbose: bool = True,
              matmul_dtype=np.float32):
    """Per-layer alpha for workload ``wl`` from full-depth greedy decode states."""
    sh = wl.shape
    L = sh.n_layers
    h = synth.geometric_hazard(wl.mean_exit, L)
    steps = wl.decode_steps if steps is None else min(steps, wl.decode_steps)
    t0 = time.time()

    def say(msg):
        if verbose:
            print(f"[calibrate {wl.name}] {msg} ({time.time() - t0:.0f}s)", flush=True)

    P0 = wl.prompt_len
    hid, w = _full_depth_states(wl, steps, calib_batch, P0, say, matmul_dtype)
    E = from_bf16_bits(w["lm_head"]).astype(matmul_dtype)
    alphas = []
    for l in range(1, L):
        hl = hid[:, :, l].reshape(-1, sh.d_model)
        T = synth.draw_unit_normal(wl.seed_weights, "head_T", l, (sh.d_model, sh.d_model)) * 0.02
        z = bf16_round(hl).astype(matmul_dtype) @ T.astype(matmul_dtype).T
        logits = (z @ E.T).astype(np.float64)
        astar = alpha_threshold(logits, wl.gamma)
        a = float(np.quantile(astar, h))
        alphas.append(a)
        say(f"layer {l}: alpha={a:.4g}")
    return {"workload": wl.name, "gamma": wl.gamma, "mean_exit": wl.mean_exit, "hazard": h,
            "samples_per_layer": int(hid.shape[0] * hid.shape[1]),
            "source": f"full-depth greedy decode, {calib_batch} prompts of {P0} tokens, {steps} steps",
            "alpha": alphas}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--criterion", choices=("head", "sts"), default="head")
    ap.add_argument("--prompt-len", type=int, default=None, help="sts only: calibration prompt length")
    args = ap.parse_args()
    wl = synth.workload(args.workload)
    if args.criterion == "sts":
        steps = wl.decode_steps if args.steps is None else min(args.steps, wl.decode_steps)
        res = calibrate_sts(wl, steps, args.batch, args.prompt_len)
        name = f"{wl.name}_sts"
    else:
        res = calibrate(wl, args.steps, args.batch)
        name = wl.name
    os.makedirs(synth.CALIB_DIR, exist_ok=True)
    path = os.path.join(synth.CALIB_DIR, f"{name}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()
