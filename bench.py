#!/usr/bin/env python3
"""Decode throughput of the KV-shared early-exit step on one MI355X.

Workload (default "8b"): Llama-3.1-8B-shaped decoder (32 layers, d 4096, 32/8
heads, head_dim 128, FFN 14336, vocab 128256) with seeded random bf16 weights,
an exit head T (4096 x 4096) after every layer, int4 group-128 exit copies,
batch 8, 1024-token uniform-random prompts, gamma 0.75 with per-layer
calibrated head scales.  The prefill is untimed; ``--warmup`` decode steps run
untimed, then ``--steps`` decode steps are timed (each step: all layers, exit
heads, exit copies, final head, tokens and exit layers back on the host).

Prints one JSON line: tokens/s, the roofline of the dominant kernel (the exit
head's vocabulary GEMV, timed with HIP events it records on its stream during a
rolled-back re-run of the timed steps), whole-step algorithmic bandwidth, the
realised exit layers, the speedup over the plain full-depth decoder and over
exit heads with unquantised exit copies (same exit layers), and the oracle's
decode speed on the host cores (a bounded sample).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak

# HBM traffic of one exit-head launch with rows on the backbone, per workload:
# the 8B shape with 8 staged rows (proj_kernel<3, 1>) and with 64 rows (the
# wide pass, wide_vocab_kernel<3>), from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs of kv_shared_exit_amd/ee_probe (profiles/*_traffic.md), each
# scaled by what the same counter reads for a 1 GiB device copy.  Valid only
# for the kernel sources it was measured on (their sha256); otherwise null.
TRAFFIC = {
    "lse": {"fetch_kib": 513397.5625, "write_kib": 62.6, "fetch_scale": 1.9999340, "write_scale": 0.9999999,
            "sources": ("ee_proj.hip", "ee_device.h", "ee_internal.h", "ee_epi.h"),
            "sources_sha256": "fe5be4b424ad6cf612d99f8526939fe985394c9b6213d38a11de3a7175df8765"},
    "wide": {"fetch_kib": 519396.8646, "write_kib": 512.0, "fetch_scale": 1.9999340, "write_scale": 0.9999999,
             "sources": ("ee_wide.hip", "ee_device.h", "ee_internal.h", "ee_epi.h"),
             "sources_sha256": "7f1965e47fe4553aa1fb250da079086f9590f5461f192770007625948b5a22f0"},
}
# the workloads whose shape (128256 x 4096) the counters were taken at
TRAFFIC_SHAPE = (128256, 4096)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sources_sha256(sources=("ee_proj.hip", "ee_device.h", "ee_internal.h", "ee_epi.h")):
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "kv_shared_exit_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def step_bytes(sh, exits, ctx, B, head_bytes=True, every=1):
    """Algorithmic HBM bytes of one decode step given the realised exit layers.

    Per layer l: bf16 weights when some row is still on the backbone (e_b >= l),
    int4 codes + bf16 scales when some row has exited (e_b < l), the exit head
    (T and E) when l < L is a check layer (a multiple of ``every``) and some
    row is on the backbone (not with the similarity criterion, which reads no
    weights); then the final LM head,
    K/V reads of every row's context, K/V writes and the embedding rows."""
    L, d, V, G = sh.n_layers, sh.d_model, sh.vocab, sh.group
    n = sh.params_per_layer()
    w_bf, w_i4 = 2 * n, n // 2 + 2 * n // G
    e = np.asarray(exits)
    tot = 0
    heads = 0
    for l in range(1, L + 1):
        A = int((e >= l).sum())
        X = B - A
        if A:
            tot += w_bf
        if X:
            tot += w_i4
        if l < L and A and l % every == 0:
            tot += (2 * d * d + 2 * V * d) if head_bytes else 0
            heads += 1
    tot += 2 * V * d
    kv_row = 2 * sh.n_kv_heads * sh.head_dim * 2
    tot += int(np.sum(ctx)) * L * kv_row + B * L * kv_row + B * d * 2
    return tot, heads


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, weights, exits, ctx, criterion="head", every=1, budget_s=30.0):
    """The oracle's decode speed on the host: decode steps of the workload's
    whole batch at its shape, over a synthetic (seeded) KV context of ``ctx``
    positions per sequence, with the exit layers the GPU's first timed step
    took (forced; the criterion is still evaluated).  BLAS threads are set to
    every core of the process's affinity set.  As many steps as fit in about
    ``budget_s`` seconds (at least one) are timed."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import model as om
    sh = wl.shape
    B = len(exits)
    cores = len(os.sched_getaffinity(0))
    orc = om.OracleModel(sh, weights, cache_f64=False)
    for l in range(int(np.min(exits)) + 1, sh.n_layers + 1):
        for name in om.LINEAR:
            orc.quantized(l, name)            # model setup, like the GPU's ee_create_model
    cache = om.KVCache(sh, B, ctx + 64)
    rng = np.random.default_rng(4242)
    kv = rng.standard_normal(cache.K[:, :, :, :ctx].shape, dtype=np.float32)
    cache.K[:, :, :, :ctx] = kv
    cache.V[:, :, :, :ctx] = kv[:, :, :, ::-1]
    del kv
    cache.lens[:B] = ctx
    toks = np.arange(1, B + 1)
    n, dt = 0, 0.0
    with threadpool_limits(limits=cores, user_api="blas"):
        info = threadpool_info()
        while n == 0 or (dt / n) * (n + 1) <= budget_s and n < 8:
            t0 = time.perf_counter()
            toks, _, _ = om.decode_step(orc, cache, toks, gamma=wl.gamma, forced=exits, criterion=criterion,
                                        check_every=every)
            dt += time.perf_counter() - t0
            n += 1
    blas = [f"{p.get('internal_api')} {p.get('version')} ({p.get('num_threads')} threads)"
            for p in info if p.get("user_api") == "blas"]
    return {"value": round(B * n / dt, 5), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"{n} decode step(s) of the batch of {B}, {sh.n_layers}-layer d{sh.d_model} shape, "
                       f"synthetic {ctx}-position KV context per sequence, exit layers of the GPU's first timed "
                       f"step forced {[int(x) for x in exits]}, "
                       f"{'similarity' if criterion == 'sts' else 'exit-head'} criterion evaluated; "
                       f"{dt:.1f} s, float64 numpy"
                       + (f" (8 steps would exceed the ~{budget_s:.0f} s sample)" if n < 8 else "")),
            "cpu_model": _cpu_model(), "blas": blas, "affinity_cores": cores}


def hbm_ceiling():
    """Measured streaming ceilings of this GPU, for the roofline fractions:
    a read-only stream of 4 GiB (the library's 16-byte non-temporal loads,
    kv_shared_exit_amd/ee_probe read, 20 launches, run as a child process;
    the grid sweeps the buffer in strided rounds), the same bytes read with
    one contiguous region per workgroup (ee_probe readc), and torch's 1 GiB
    device-to-device copy (read + write, 10 launches timed with events on the
    current stream)."""
    import subprocess
    import torch
    out = {}
    probe = os.path.join(ROOT, "kv_shared_exit_amd", "ee_probe")
    if os.path.exists(probe):
        for key, mode, kind in (("read", "read", "4 GiB read stream, strided rounds (ee_probe read, 20 launches)"),
                                ("read_regions", "readc",
                                 "4 GiB read, one contiguous region per workgroup (ee_probe readc, 20 launches)")):
            r = subprocess.run([probe, mode, "4096", "20"], capture_output=True, text=True, timeout=120)
            if r.returncode == 0 and "GB/s" in r.stdout:
                gbs = float(r.stdout.strip().split(",")[-1].split()[0])
                out[key] = {"kind": kind, "GBps": gbs, "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    gbs = 2 * x.numel() * 4 / (ms * 1e-3) / 1e9
    del x, y
    out["copy"] = {"kind": "1 GiB device copy, torch (read + write)", "GBps": round(gbs, 1),
                   "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def prefill_flops(sh, B, P, chunk):
    """Algorithmic flops of the prefill of B sequences of P positions given in
    calls of `chunk` positions: every projection over every position (2 flops
    per weight per position), causal attention (scores and the weighted sum,
    4 hd flops per (query, visible key) per q head) and the LM head of each
    call's last position."""
    L, d, V, hd, H = sh.n_layers, sh.d_model, sh.vocab, sh.head_dim, sh.n_heads
    proj = 2 * B * P * sh.params_per_layer() * L
    ctx = np.arange(1, P + 1, dtype=np.float64).sum()      # visible keys summed over the positions
    attn = 4 * hd * H * ctx * B * L
    calls = (P + chunk - 1) // chunk
    head = 2 * B * V * d * calls
    return proj + attn + head


def prefill(api, model, cache, prompts, stream, t0, chunk=512):
    """Prefill in chunks of positions (the library appends each chunk after the
    cached positions), logging progress on long prompts; with the prefill's
    sequence-level exit the whole prompt is one call (the decision takes the
    minimum over all of its tokens).  Returns the exit layers of the last call."""
    P = prompts.shape[1]
    if model.cfg.prefill_exit:
        chunk = P
    ex = None
    for p0 in range(0, P, chunk):
        _, ex = api.prefill(model, cache, prompts[:, p0:p0 + chunk], stream=stream, exits=True)
        if P > chunk:
            log(f"prefill positions {min(p0 + chunk, P)}/{P} ({time.time() - t0:.0f}s)")
    return ex


def baselines(api, wl, weights, dev, stream, exits, W, K2, ms_main, criterion=0, thresholds=None, every=1,
              rule=0):
    """The method against the decoders it replaces, on the same prompts and
    weights, each timed over K2 graph-replayed steps after W warm-up steps:
    (i) the plain decoder at full depth without exit heads (EE_EXIT_NONE);
    (ii) exit heads with unquantised exit copies (EE_EXIT_BF16) and the exit
    layers the timed run took, step by step (forced).  speedup = baseline time
    per step / the method's time per step."""
    import torch
    from kv_shared_exit_amd import _binding as Bd
    sh, B, P = wl.shape, wl.batch, wl.prompt_len
    S = P + W + K2 + 1
    import synth
    prompts = synth.make_prompts(wl)
    res = {}
    for name, mode in (("full_depth_no_heads", Bd.EE_EXIT_NONE), ("bf16_exit_copies_same_exits", Bd.EE_EXIT_BF16)):
        m = api.Model(sh, dev, gamma=wl.gamma if thresholds is None else thresholds, exit_mode=mode,
                      max_batch=B, max_positions=S, criterion=criterion, check_every=every, exit_rule=rule)
        c = api.KVCache(m, B, S)
        try:
            prefill(api, m, c, prompts, stream, time.time())
            forced = (lambda s_: exits[s_ % len(exits)]) if mode == Bd.EE_EXIT_BF16 else (lambda s_: None)
            for s_ in range(W):
                api.decode_step(m, c, B, forced=forced(s_), stream=stream)
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            for s_ in range(K2):
                api.decode_step(m, c, B, forced=forced(s_), stream=stream)
            torch.cuda.synchronize()
            res[name + "_ms_per_step"] = round(1e3 * (time.perf_counter() - t_start) / K2, 4)
        finally:
            c.close()
            m.close()
    return {"steps": K2, "method_ms_per_step": round(ms_main, 4), **res,
            "vs_full_depth_no_heads": round(res["full_depth_no_heads_ms_per_step"] / ms_main, 4),
            "vs_bf16_exit_copies_same_exits": round(res["bf16_exit_copies_same_exits_ms_per_step"] / ms_main, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true",
                    help="do not time the exit-head launches (no roofline figure)")
    ap.add_argument("--criterion", choices=("head", "sts"), default="head",
                    help="exit criterion: the exit head (default) or River-LLM's state transition "
                         "similarity with the workload's calibrated thresholds (secondary line)")
    ap.add_argument("--exit-rule", choices=("sequence", "batch-min"), default="sequence",
                    help="per-sequence exits (default) or River-LLM's batch minimum (secondary line)")
    ap.add_argument("--check-every", type=int, default=1,
                    help="evaluate the exit criterion only after every N-th layer (secondary line)")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="sampled decoding with AdaDecode's verification at this temperature (secondary "
                         "line; 0: greedy)")
    ap.add_argument("--prefill-exit", action="store_true",
                    help="River-LLM's sequence-level exit in the prefill (with --criterion sts)")
    ap.add_argument("--no-baselines", action="store_true",
                    help="skip the full-depth and bf16-exit-copy comparison runs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the early-exit decode step is data-parallel "
              "(every sequence is independent) and the library runs on one MI355X; "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from kv_shared_exit_amd import api

    wl = synth.workload(args.workload)
    sh = wl.shape
    B, P = wl.batch, wl.prompt_len
    K = args.steps if args.steps is not None else wl.decode_steps - args.warmup
    W = args.warmup
    S = P + W + K + 1
    from kv_shared_exit_amd import _binding as Bd
    sts = args.criterion == "sts"
    crit = Bd.EE_CRIT_STS if sts else Bd.EE_CRIT_HEAD
    thresholds = wl.gamma
    if sts:
        thresholds = synth.load_tau(wl, batch_min=args.exit_rule == "batch-min")
        if thresholds is None:
            print(f"no similarity thresholds for {wl.name} (synth/calibration/{wl.name}_sts.json)", file=sys.stderr)
            sys.exit(2)
    if args.prefill_exit and not sts:
        print("--prefill-exit needs --criterion sts (the prefill's exit uses the token similarities)", file=sys.stderr)
        sys.exit(2)
    alpha = synth.load_alpha(wl)
    # a calibrated workload without calibrated exit-head scales (the 34B shape:
    # its float64 oracle does not fit host memory) runs the exit layers of its
    # target distribution as forced exits; the heads are still computed
    target = alpha is None and wl.policy == "calibrated" and not sts
    if target:
        log("no calibration file: exit layers drawn from the target distribution (forced), heads computed")
    t0 = time.time()
    weights = synth.make_weights(sh, wl.seed_weights, alpha=alpha)
    if sts:  # the similarity criterion reads no head weights
        for lw in weights["layers"]:
            lw.pop("head_T", None)
    log(f"weights drawn ({time.time() - t0:.0f}s)")
    dev = api.upload_weights(weights)
    every = max(1, args.check_every)
    rule = Bd.EE_RULE_BATCH_MIN if args.exit_rule == "batch-min" else Bd.EE_RULE_SEQUENCE
    model = api.Model(sh, dev, gamma=thresholds, max_batch=B, max_positions=S, criterion=crit, check_every=every,
                      exit_rule=rule, temperature=args.temperature, sample_seed=wl.seed_prompts,
                      prefill_exit=args.prefill_exit)
    cache = api.KVCache(model, B, S)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    log(f"model ready ({time.time() - t0:.0f}s)")
    prompts = synth.make_prompts(wl)
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    pexits = prefill(api, model, cache, prompts, stream, t0)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - tp0
    pf_flops = prefill_flops(sh, B, P, P if args.prefill_exit else 512)
    log(f"prefill {B}x{P} done in {prefill_s:.3f}s ({time.time() - t0:.0f}s)")

    exits, toks = [], []

    def step(s, tokens=None):
        f = (synth.make_forced_exits(wl, s) if wl.policy == "forced" else
             synth.make_target_exits(wl, s) if target else None)
        return api.decode_step(model, cache, B, tokens=tokens, forced=f, stream=stream)

    last = None
    for s in range(W):
        last, _ = step(s)
    torch.cuda.synchronize()
    ctx0 = cache.lengths()[:B].copy()
    tok_in0 = last.copy()
    # timed region: the production path (each step replays its captured graph)
    torch.cuda.synchronize()
    step_ms = []
    t_start = time.perf_counter()
    for s in range(K):
        ts = time.perf_counter()
        t, e = step(W + s)     # returns after the step's outputs are on the host
        step_ms.append(1e3 * (time.perf_counter() - ts))
        toks.append(t.copy())
        exits.append(e.copy())
    torch.cuda.synchronize()
    t_el = time.perf_counter() - t_start
    log(f"timed {K} steps in {t_el:.3f}s")

    # the same K steps once more, rolled back and re-run with the same inputs,
    # each exit-head launch timed by events it records itself (profiled steps
    # launch their kernels one by one); the decisions must repeat exactly
    n_launch, head_ms = 0, 0.0
    if not args.no_profile and not sts:
        cache.rollback(-1, K)
        model.profile(True)
        tin = tok_in0
        for s in range(K):
            t, e = step(W + s, tokens=tin)
            if not (np.array_equal(t, toks[s]) and np.array_equal(e, exits[s])):
                raise RuntimeError(f"profiled re-run of step {s} differs from the timed run")
            tin = t
        torch.cuda.synchronize()
        n_launch, head_ms = model.profile_read(0)
        model.profile(False)
        log(f"profiled re-run: {n_launch} exit-head launches, {head_ms:.2f} ms")

    exits = np.stack(exits)
    total_bytes = 0
    head_launches = 0
    for s in range(K):
        ctx = ctx0 + s + 1
        b, h = step_bytes(sh, exits[s], ctx, B, head_bytes=not sts, every=every)
        total_bytes += b
        head_launches += h
    # dominant kernel: the exit head's vocabulary GEMV.  It is launched after
    # every layer l < L; a launch reads E (V x d bf16) and the staged rows when
    # some row is still on the backbone, and returns at once otherwise.  The
    # roofline figure is the launches' algorithmic bytes over their summed
    # duration (= mean bytes per launch / mean launch time).
    head_bytes_total = 0
    head_flops_total = 0
    for s_ in range(K):
        for l in range(every, sh.n_layers, every):
            a_rows = int((exits[s_] >= l).sum())
            if a_rows:
                head_bytes_total += 2 * sh.vocab * sh.d_model + 2 * sh.d_model * a_rows
                head_flops_total += 2 * sh.vocab * sh.d_model * a_rows
    avg_ms = head_ms / max(n_launch, 1)
    head_bytes = head_bytes_total / n_launch if n_launch else 0.0
    achieved = head_bytes_total / (head_ms * 1e-3) / 1e9 if n_launch else 0.0
    # measured HBM traffic per launch, averaged like the algorithmic bytes (a
    # launch without rows reads nothing)
    traffic = None
    # batches above 8 run every exit head on the wide pass, batches up to 8 on
    # the 8-row pass: each launch with work takes its kernel's measured bytes
    def measured(kind):
        tr = TRAFFIC[kind]
        if kernel_sources_sha256(tr["sources"]) != tr["sources_sha256"]:
            return None
        return (tr["fetch_kib"] * tr["fetch_scale"] + tr["write_kib"] * tr["write_scale"]) * 1024
    if (sh.vocab, sh.d_model) == TRAFFIC_SHAPE and not sts and args.temperature == 0 and n_launch:
        tot = 0.0
        for s_ in range(K):
            for l in range(every, sh.n_layers, every):
                a_rows = int((exits[s_] >= l).sum())
                if a_rows:
                    t_ = measured("wide" if B > 8 else "lse")
                    tot = None if t_ is None or tot is None else tot + t_
        traffic = None if tot is None else round(tot / n_launch)

    copy_probe = None
    if args.copy_probe:
        x = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        copy_probe = {"bytes_read": x.numel() * 4, "bytes_written": y.numel() * 4}

    if args.temperature > 0:
        head_kernel = "exit-head vocabulary GEMV with the draft's draw (proj_kernel<6, 1>)"
    elif B > 8:
        head_kernel = "exit-head vocabulary GEMV (wide_vocab_kernel<3>, any number of rows on the backbone)"
    else:
        head_kernel = "exit-head vocabulary GEMV (proj_kernel<3, 1>)"
    hist = np.bincount(exits.reshape(-1), minlength=sh.n_layers + 1)[1:]
    mean_exit = float(exits.mean())
    out = {
        "metric": "decode tokens/s at 1 MI355X (8B shape, b=8) + achieved HBM GB/s fraction",
        "value": round(B * K / t_el, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(1e3 * t_el / K, 4),
        "step_ms": {"median": round(float(np.median(step_ms)), 4),
                    "p99": round(float(np.percentile(step_ms, 99)), 4),
                    "min": round(float(np.min(step_ms)), 4), "max": round(float(np.max(step_ms)), 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {sh.n_layers} layers d{sh.d_model} "
                               f"{sh.n_heads}/{sh.n_kv_heads} heads hd{sh.head_dim} F{sh.d_ff} "
                               f"V{sh.vocab}, int4 G{sh.group} exit copies, batch {B}, "
                               f"{P}-token prompts, gamma {wl.gamma}",
                   "global_batch": B, "seq_len": P, "decode_steps": K, "parallelism": "none"},
        "roofline": {"bound": "hbm", "kernel": head_kernel,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "launches": n_launch, "launches_with_work": head_launches,
                     "avg_us": round(1e3 * avg_ms, 2), "bytes_per_launch": int(head_bytes)},
        "step": {"algorithmic_GB": round(total_bytes / K / 1e9, 3),
                 "GBps": round(total_bytes / t_el / 1e9, 1),
                 "frac": round(total_bytes / t_el / 1e9 / HBM_PEAK_GBS, 4),
                 "mean_exit_layer": round(mean_exit, 3),
                 "exit_hist": hist.tolist(),
                 "head_launches_per_step": round(head_launches / K, 2)},
        "cpu_baseline": None,
        "prefill": {"seconds": round(prefill_s, 3), "positions": P, "batch": B,
                    "positions_per_s": round(B * P / prefill_s, 1),
                    "chunk": P if args.prefill_exit else min(P, 512),
                    "mfma": {"dtype": "bf16", "achieved": round(pf_flops / prefill_s / 1e12, 1),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(pf_flops / prefill_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
                    "exit_layers": None if pexits is None else [int(x) for x in pexits]},
    }
    if wl.name != "8b":
        out["metric"] = out["metric"].replace("(8B shape, b=8)", f"({wl.name} shape, b={B})")
    if B > 8 and n_launch:
        # more than 8 rows run the exit head's vocabulary GEMV on matrix cores
        # (bf16 MFMA): its algorithmic flops (2 V d per row on the backbone)
        # over the same launch times as the roofline
        tf = head_flops_total / (head_ms * 1e-3) / 1e12
        out["mfma"] = {"kernel": "wide exit-head vocabulary pass (wide_vocab_kernel<3>)", "dtype": "bf16",
                       "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    if wl.policy == "forced":
        out["config"]["workload"] += (f", exit layers forced uniform in [{wl.forced_lo}, {wl.forced_hi}] "
                                      f"per sequence and step (heads computed)")
    elif target:
        out["config"]["workload"] += (f", exit layers forced from the target distribution (truncated geometric, "
                                      f"mean {wl.mean_exit}; heads computed, no calibrated scales)")
    if copy_probe:
        out["copy_probe"] = copy_probe
    cache.close()
    model.close()
    if rule == Bd.EE_RULE_BATCH_MIN:
        out["metric"] += ", batch-minimum exits"
        out["config"]["workload"] += ", batch-minimum exit rule"
    if args.prefill_exit:
        out["config"]["workload"] += ", sequence-level exit in the prefill (minimum token similarity)"
    if args.temperature > 0:
        out["metric"] += f", sampled (temperature {args.temperature}, verified drafts)"
        out["config"]["workload"] += (f", sampled decoding at temperature {args.temperature} with AdaDecode's "
                                      f"verification of the exit-layer drafts")
    if every > 1:
        out["metric"] += f", criterion every {every} layers"
        out["config"]["workload"] += f", criterion evaluated after every {every}th layer"
    if sts:  # no exit-head GEMV runs: the whole step is the measured unit
        step_gbs = total_bytes / t_el / 1e9
        out["metric"] = out["metric"].replace("(8B shape, b=8)", "(8B shape, b=8), state-transition-similarity exits")
        out["config"]["workload"] += ", exit criterion: state transition similarity (calibrated tau)"
        out["roofline"] = {"bound": "hbm", "kernel": "whole decode step (no exit-head GEMV under this criterion)",
                           "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(step_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    out["hbm_ceiling"] = hbm_ceiling()
    if not args.no_baselines:
        out["speedup"] = baselines(api, wl, weights, dev, stream, exits, W, min(K, 40), 1e3 * t_el / K,
                                   criterion=crit, thresholds=thresholds, every=every, rule=rule)
        log(f"baselines done ({time.time() - t0:.0f}s)")
    del dev
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, weights, exits[0], P, criterion=args.criterion, every=every)
        log(f"cpu baseline done ({time.time() - t0:.0f}s)")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
