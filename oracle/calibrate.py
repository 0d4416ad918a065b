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

Samples come from a layer-major prefill of seeded calibration prompts
(positions in the same range the workload decodes), at full depth with the
backbone weights.  The unit-scale logits use T drawn at standard deviation
0.02 without bf16 rounding; the realised exit distribution is therefore close
to, not exactly, the target.  Parity unpinned: this only chooses inputs.

Usage: python -m oracle.calibrate <workload> [--samples N]
writes synth/calibration/<workload>.json.
"""
from __future__ import annotations

import argparse
import json
import os
import time

import numpy as np

import synth
from .model import OracleModel, KVCache, prefill
from .numerics import bf16_round


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


def calibrate(wl, samples: int | None = None, calib_batch: int = 1, verbose: bool = True):
    sh = wl.shape
    L = sh.n_layers
    h = synth.geometric_hazard(wl.mean_exit, L)
    # positions of the samples: the decode range of the workload
    P0 = wl.prompt_len
    n_pos = min(wl.decode_steps + 1, samples or (wl.decode_steps + 1))
    Pc = P0 + n_pos
    t0 = time.time()
    w = synth.make_weights(sh, wl.seed_weights)
    m = OracleModel(sh, w, exit_mode="bf16", cache_f64=False)
    cache = KVCache(sh, calib_batch, Pc)
    prompts = synth.make_prompts(wl, batch=calib_batch, length=Pc, seed=wl.seed_calib)
    _, info = prefill(m, cache, prompts, trace=True)
    hid = info["hidden"][:, P0:Pc]                            # [Bc, n_pos, L+1, d]
    if verbose:
        print(f"[calibrate {wl.name}] prefill of {calib_batch}x{Pc} done in {time.time()-t0:.0f}s",
              flush=True)
    E = m.lm_head
    alphas = []
    for l in range(1, L):
        hl = hid[:, :, l].reshape(-1, sh.d_model)
        T = synth.draw_unit_normal(wl.seed_weights, "head_T", l, (sh.d_model, sh.d_model))
        T = T.astype(np.float64) * 0.02
        z = bf16_round(hl) @ T.T
        logits = z @ E.T
        astar = alpha_threshold(logits, wl.gamma)
        a = float(np.quantile(astar, h))
        alphas.append(a)
        if verbose:
            print(f"[calibrate {wl.name}] layer {l}: alpha={a:.4g} ({time.time()-t0:.0f}s)", flush=True)
    return {"workload": wl.name, "gamma": wl.gamma, "mean_exit": wl.mean_exit, "hazard": h,
            "samples_per_layer": int(hid.shape[0] * hid.shape[1]),
            "positions": [P0, Pc], "alpha": alphas}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("--samples", type=int, default=None)
    ap.add_argument("--batch", type=int, default=1)
    args = ap.parse_args()
    wl = synth.workload(args.workload)
    res = calibrate(wl, args.samples, args.batch)
    os.makedirs(synth.CALIB_DIR, exist_ok=True)
    path = os.path.join(synth.CALIB_DIR, f"{wl.name}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()
