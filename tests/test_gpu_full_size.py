"""GPU checks at the benchmark's full size: the 8B decoder shape (32 layers,
d 4096, 32/8 heads, F 14336, V 128256, int4 G128 copies) with batch 8, the
launch configuration bench.py times.

The oracle cannot run whole generations at this size, so the comparisons are
sampled (one sequence, a few positions; by batch independence a sequence run
alone by the oracle equals the same sequence inside the GPU's batch), and the
rest are properties that hold at any size:
  * full depth (gamma > 1, nobody exits): sequence 0's prefill logits, its
    decode step's hidden state after every layer, logits, token and its K/V
    against the oracle run without exit heads (heads cannot change a step in
    which nobody exits);
  * exit after layer 1 (every row runs layers 2..L on the int4 copies): the
    hidden states after layers 1 and 2 against the oracle's first two layers
    (the later layers do not influence them), and every row's exit-head
    probability after layer 1 (the vocabulary GEMV over V = 128256 in its
    decode-step grid, and the decision's merge of its partials) within the
    bound derived from the measured error of the head's input;
  * half the batch forced out after layer 1 on a three-layer slice: layers 2
    and 3 run backbone rows and exited rows in the same launches (the mixed
    split of the workgroups the benchmark runs), hidden states, K/V and the
    exit-head probabilities of a row of each kind against the oracle;
  * int4 copies bit-exact for sampled rows of sampled layers;
  * at the benchmark's prompt length: graph replay equals launching the
    kernels one by one (tokens, exit layers, K/V), and every written KV slot
    was written exactly once;
  * two layers at the exact widths of the 1B and 34B workloads (batch 2 and
    4), half the rows forced out after layer 1 so that layer 2 runs the int4
    copies at K = 8192 / 22016 and head_dim 64 next to the backbone rows;
  * the batch-64 wide passes at the 8B widths at full depth, all rows exited,
    and half the rows exited (both formats in one wide launch);
  * the prefill's matrix-core path at the 8B widths (two layers, 520 prompt
    positions in the benchmark's 512-position calls): K/V of every position
    and the last position's logits against the oracle, at full depth and with
    every sequence leaving after layer 1 (layer 2 on the int4 G128 copies).
"""
import dataclasses

import numpy as np
import pytest

import synth
from parity import head_lnp_bound
from oracle import model as om
from oracle.numerics import from_bf16_bits
from oracle.quant import quantize_int4

pytestmark = pytest.mark.gpu

SH = synth.LLAMA8B
B = 8
TOL = 2e-2


def maxrel(a, r):
    a = np.asarray(a, np.float64)
    r = np.asarray(r, np.float64)
    return float(np.abs(a - r).max() / max(np.abs(r).max(), 1e-30))


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_shared_exit_amd import api
    wl = synth.workload("8b")
    w = synth.make_weights(SH, wl.seed_weights, alpha=synth.load_alpha(wl))
    dev = api.upload_weights(w)
    torch.cuda.synchronize()
    yield api, w, dev
    del dev


def _prompts(P):
    return np.random.default_rng(77).integers(0, SH.vocab, (B, P)).astype(np.int32)


def test_full_depth_sequence_matches_oracle(env):
    api, w, dev = env
    P = 3
    prompts = _prompts(P)
    model = api.Model(SH, dev, gamma=2.0, max_batch=B, max_positions=P + 2)
    cache = api.KVCache(model, B, P + 2, track=True)
    try:
        tg, lg = api.prefill(model, cache, prompts, logits=True)
        dbg = {"logits": None, "hidden": None, "p": None}
        tok_in = tg.copy()
        t1, e1 = api.decode_step(model, cache, B, tokens=tok_in, debug=dbg)
        assert np.all(e1 == SH.n_layers)
        k_gpu = {l: cache.read(l, 0, 0, P + 1) for l in (1, 16, 32)}
    finally:
        cache.close()
        model.close()

    orc = om.OracleModel(SH, w, cache_f64=True)   # widened once, used by both passes
    oc = om.KVCache(SH, 1, P + 2)
    to, info = om.prefill(orc, oc, prompts[:1])
    e = maxrel(lg[0], info["logits"][0])
    assert e <= TOL, f"prefill logits maxrel {e:.3g}"
    band = max(1e-2, 2 * float(np.abs(lg[0].astype(np.float64) - info["logits"][0]).max()))
    if info["gap"][0] > band:
        assert tg[0] == to[0]
    t2, e2, io = om.decode_step(orc, oc, tok_in[:1], trace=True, heads=False)
    for l in range(SH.n_layers + 1):
        e = maxrel(dbg["hidden"][0, l], io["hidden"][0, l])
        assert e <= TOL, f"hidden after layer {l}: maxrel {e:.3g}"
    e = maxrel(dbg["logits"][0], io["logits"][0])
    assert e <= TOL, f"decode logits maxrel {e:.3g}"
    band = max(1e-2, 2 * float(np.abs(dbg["logits"][0].astype(np.float64) - io["logits"][0]).max()))
    if io["gap"][0] > band:
        assert t1[0] == t2[0]
    for l, (k, v) in k_gpu.items():
        kr = oc.K[l - 1, 0, :, :P + 1].transpose(1, 0, 2)
        vr = oc.V[l - 1, 0, :, :P + 1].transpose(1, 0, 2)
        # K/V of layer l are linear maps of the hidden state entering it: their
        # max-relative error follows that state's measured divergence (rounding
        # flips of earlier layers grow with depth in this random-weight decoder)
        allow = kv_allowance(dbg["hidden"][0, l - 1], io["hidden"][0, l - 1])
        ek, ev = maxrel(from_bf16_bits(k), kr), maxrel(from_bf16_bits(v), vr)
        print(f"KV layer {l}: maxrel K {ek:.4f} V {ev:.4f} allowed {allow:.4f}", flush=True)
        assert ek <= allow and ev <= allow, f"KV layer {l}: {ek:.4f} {ev:.4f} > {allow:.4f}"


def kv_allowance(h_gpu, h_orc):
    """Allowed max-relative error of a layer's K/V given the measured error of
    the hidden state entering the layer: the stated 2e-2, or, when the input
    has diverged further, 1.5 times its norm-relative error (the largest
    output error of a random linear map over its largest output follows the
    norm-relative error of its input, within the spread of Gaussian maxima)
    plus 2^-8 (one rounding of RoPE's output)."""
    a = np.asarray(h_gpu, np.float64)
    r = np.asarray(h_orc, np.float64)
    nrel = float(np.linalg.norm(a - r) / max(np.linalg.norm(r), 1e-30))
    return max(TOL, 1.5 * nrel + 2.0 ** -8)


def test_exit_after_layer_one_runs_int4_copies(env):
    api, w, dev = env
    P = 2
    prompts = _prompts(P)
    model = api.Model(SH, dev, gamma=0.75, max_batch=B, max_positions=P + 2)
    cache = api.KVCache(model, B, P + 2, track=True)
    try:
        tg = api.prefill(model, cache, prompts)
        dbg = {"hidden": None, "p": None}
        t1, e1 = api.decode_step(model, cache, B, tokens=tg, forced=np.ones(B, np.int32), debug=dbg)
        np.testing.assert_array_equal(e1, np.ones(B, np.int32))
        assert np.all(np.isnan(dbg["p"][:, 1:])), "heads after the exit layer must not run"
    finally:
        cache.close()
        model.close()
    # the oracle's first two layers: layer 1 on the backbone, layer 2 on its int4 copy
    sh2 = dataclasses.replace(SH, n_layers=2)
    w2 = {"tok_emb": w["tok_emb"], "lm_head": w["lm_head"], "final_norm": w["final_norm"],
          "layers": w["layers"][:2]}
    orc = om.OracleModel(sh2, w2, cache_f64=False)
    oc = om.KVCache(sh2, B, P + 2)
    om.prefill(orc, oc, prompts)
    _, eo, io = om.decode_step(orc, oc, tg, forced=np.ones(B), trace=True)
    assert np.all(eo == 1)
    for b in range(B):
        for l in range(3):
            e = maxrel(dbg["hidden"][b, l], io["hidden"][b, l])
            assert e <= TOL, f"b={b} hidden after layer {l}: maxrel {e:.3g}"
        # the exit head after layer 1: V = 128256 rows of E, the decode step's grid of partials
        bound = head_lnp_bound(orc, 1, dbg["hidden"][b, 1], io["hidden"][b, 1])
        dl = abs(np.log(float(dbg["p"][b, 0])) - np.log(float(io["p"][b, 0])))
        print(f"b={b} p gpu {dbg['p'][b, 0]:.6g} oracle {io['p'][b, 0]:.6g} |d ln p| {dl:.3g} bound {bound:.3g}",
              flush=True)
        assert dl <= bound, f"b={b}: exit-head ln p error {dl:.3g} > bound {bound:.3g}"


def test_mixed_formats_in_one_launch_at_full_width(env):
    """Rows 0-3 forced out after layer 1, rows 4-7 on the backbone (gamma 2):
    layers 2 and 3 of an 8B slice serve both row lists in each projection
    launch.  Rows 0 (int4 copies) and 4 (backbone) against the oracle: hidden
    states after every layer, K/V of both layers, and the exit-head
    probabilities after layers 1 (both rows) and 2 (row 4)."""
    api, w, dev = env
    P = 2
    sh3 = dataclasses.replace(SH, n_layers=3)
    w3 = {"tok_emb": w["tok_emb"], "lm_head": w["lm_head"], "final_norm": w["final_norm"],
          "layers": [dict(lw) for lw in w["layers"][:3]]}
    del w3["layers"][2]["head_T"]
    dev3 = {"tok_emb": dev["tok_emb"], "lm_head": dev["lm_head"], "final_norm": dev["final_norm"],
            "layers": dev["layers"][:3]}
    prompts = _prompts(P)
    forced = np.array([1, 1, 1, 1, 0, 0, 0, 0], np.int32)
    model = api.Model(sh3, dev3, gamma=2.0, max_batch=B, max_positions=P + 2)
    cache = api.KVCache(model, B, P + 2, track=True)
    try:
        tg = api.prefill(model, cache, prompts)
        dbg = {"hidden": None, "p": None, "logits": None}
        t1, e1 = api.decode_step(model, cache, B, tokens=tg, forced=forced, debug=dbg)
        np.testing.assert_array_equal(e1, np.where(forced > 0, 1, 3))
        kv = {(l, b): cache.read(l, b, 0, P + 1) for l in (2, 3) for b in (0, 4)}
        assert np.all(cache.occupancy()[:, :B, :P + 1] == 1)
    finally:
        cache.close()
        model.close()
    orc = om.OracleModel(sh3, w3, cache_f64=False)
    oc = om.KVCache(sh3, 2, P + 2)
    om.prefill(orc, oc, prompts[[0, 4]])
    _, eo, io = om.decode_step(orc, oc, tg[[0, 4]], gamma=2.0, forced=forced[[0, 4]], trace=True)
    np.testing.assert_array_equal(eo, [1, 3])
    for i, b in enumerate((0, 4)):
        for l in range(4):
            e = maxrel(dbg["hidden"][b, l], io["hidden"][i, l])
            assert e <= TOL, f"b={b} hidden after layer {l}: maxrel {e:.3g}"
        e = maxrel(dbg["logits"][b], io["logits"][i])
        assert e <= TOL, f"b={b} logits maxrel {e:.3g}"
        for l in (2, 3):
            k, v = kv[(l, b)]
            kr = oc.K[l - 1, i, :, :P + 1].transpose(1, 0, 2)
            vr = oc.V[l - 1, i, :, :P + 1].transpose(1, 0, 2)
            assert maxrel(from_bf16_bits(k), kr) <= TOL and maxrel(from_bf16_bits(v), vr) <= TOL, f"b={b} KV {l}"
        np.testing.assert_array_equal(np.isnan(dbg["p"][b]), np.isnan(io["p"][i]))
        for l in np.nonzero(np.isfinite(io["p"][i]))[0] + 1:
            bound = head_lnp_bound(orc, int(l), dbg["hidden"][b, l], io["hidden"][i, l])
            dl = abs(np.log(float(dbg["p"][b, l - 1])) - np.log(float(io["p"][i, l - 1])))
            assert dl <= bound, f"b={b} layer {l}: ln p error {dl:.3g} > bound {bound:.3g}"


def test_int4_copies_sampled_rows_bit_exact(env):
    api, w, dev = env
    model = api.Model(SH, dev, max_batch=B, max_positions=4)
    try:
        rng = np.random.default_rng(5)
        for l in (2, 17, 32):
            for name in ("wq", "wv", "wo", "w_gate", "w_down"):
                N, K = SH.linear_shapes()[name]
                for row0 in sorted(set(rng.integers(0, N - 16, 3).tolist() + [N - 16])):
                    codes, scales = model.exit_weights(l, name, row0, 16)
                    ref = from_bf16_bits(w["layers"][l - 1][name][row0:row0 + 16])
                    q, s = quantize_int4(ref, SH.group)
                    np.testing.assert_array_equal(codes, q, err_msg=f"layer {l} {name} rows {row0}..")
                    np.testing.assert_array_equal(from_bf16_bits(scales), s)
    finally:
        model.close()


def test_bench_configuration_graph_equals_eager_and_slots_written_once(env):
    import torch
    api, w, dev = env
    wl = synth.workload("8b")
    P, steps = wl.prompt_len, 3
    prompts = synth.make_prompts(wl)
    model = api.Model(SH, dev, gamma=wl.gamma, max_batch=B, max_positions=P + steps + 1)
    cache = api.KVCache(model, B, P + steps + 1, track=True)
    stream = torch.cuda.Stream()
    try:
        tok = api.prefill(model, cache, prompts, stream=stream)
        graph_out, tin = [], tok.copy()
        for s in range(steps):          # no debug outputs: the captured graph is replayed
            t, e = api.decode_step(model, cache, B, tokens=tin, stream=stream)
            graph_out.append((t.copy(), e.copy()))
            tin = t
        kv_graph = [cache.read(l, b, P, steps) for l in (1, 8, 32) for b in (0, 7)]
        occ = cache.occupancy()
        assert np.all(occ[:, :B, :P + steps] == 1) and np.all(occ[:, :B, P + steps:] == 0)
        cache.rollback(-1, steps)
        tin = tok.copy()
        for s in range(steps):          # with debug outputs: kernels launched one by one
            t, e = api.decode_step(model, cache, B, tokens=tin, stream=stream, debug={"p": None})
            np.testing.assert_array_equal(t, graph_out[s][0])
            np.testing.assert_array_equal(e, graph_out[s][1])
            tin = t
        kv_eager = [cache.read(l, b, P, steps) for l in (1, 8, 32) for b in (0, 7)]
        for (kg, vg), (ke, ve) in zip(kv_graph, kv_eager):
            np.testing.assert_array_equal(kg, ke)
            np.testing.assert_array_equal(vg, ve)
        assert np.all(cache.occupancy()[:, :B, :P + steps] == 1)
    finally:
        cache.close()
        model.close()


@pytest.mark.parametrize("name,batch", [("1b", 2), ("34b", 4)])
def test_layer_widths_of_other_workloads(name, batch):
    """Two layers with the exact widths of the 1B (d 2048, 32/8 heads of 64,
    F 8192, V 128256) and 34B (d 8192, 64/8 heads of 128, F 22016, V 32000)
    workloads: the kernels see the same shapes as in the full models (depth
    does not change any launch).  The first half of the rows is forced out
    after layer 1, so layer 2 runs the int4 copies (K = 8192 or 22016 in the
    down projection; head_dim 64 for 1B) in the same launches as the backbone
    rows of the second half.  The first and the last sequence against the
    oracle (hidden states, logits, token, K/V, the exit head's probability
    after layer 1); int4 copies bit-exact on sampled rows."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_shared_exit_amd import api
    wl = synth.workload(name)
    sh = dataclasses.replace(wl.shape, n_layers=2)
    w = synth.make_weights(sh, wl.seed_weights)
    P = 3
    prompts = np.random.default_rng(78).integers(0, sh.vocab, (batch, P)).astype(np.int32)
    dev = api.upload_weights(w)
    forced = np.array([1] * (batch // 2) + [0] * (batch - batch // 2), np.int32)
    model = api.Model(sh, dev, gamma=2.0, max_batch=batch, max_positions=P + 2)
    cache = api.KVCache(model, batch, P + 2, track=True)
    try:
        tg, lg = api.prefill(model, cache, prompts, logits=True)
        dbg = {"logits": None, "hidden": None, "p": None}
        t1, e1 = api.decode_step(model, cache, batch, tokens=tg, forced=forced, debug=dbg)
        np.testing.assert_array_equal(e1, np.where(forced > 0, 1, sh.n_layers))
        k_gpu = {(l, b): cache.read(l, b, 0, P + 1) for l in (1, 2) for b in (0, batch - 1)}
        codes, scales = model.exit_weights(2, "w_down", 64, 16)
    finally:
        cache.close()
        model.close()
    q, s_ = quantize_int4(from_bf16_bits(w["layers"][1]["w_down"][64:80]), sh.group)
    np.testing.assert_array_equal(codes, q)
    np.testing.assert_array_equal(from_bf16_bits(scales), s_)
    orc = om.OracleModel(sh, w, cache_f64=True)
    rows = [0, batch - 1]
    oc = om.KVCache(sh, 2, P + 2)
    to, info = om.prefill(orc, oc, prompts[rows])
    t2, e2, io = om.decode_step(orc, oc, tg[rows], gamma=2.0, forced=forced[rows], trace=True)
    np.testing.assert_array_equal(e2, e1[rows])
    for i, b in enumerate(rows):
        assert maxrel(lg[b], info["logits"][i]) <= TOL
        for l in range(sh.n_layers + 1):
            e = maxrel(dbg["hidden"][b, l], io["hidden"][i, l])
            assert e <= TOL, f"{name} b={b}: hidden after layer {l}: maxrel {e:.3g}"
        e = maxrel(dbg["logits"][b], io["logits"][i])
        assert e <= TOL, f"{name} b={b}: logits maxrel {e:.3g}"
        band = max(1e-2, 2 * float(np.abs(dbg["logits"][b].astype(np.float64) - io["logits"][i]).max()))
        if io["gap"][i] > band:
            assert t1[b] == t2[i]
        bound = head_lnp_bound(orc, 1, dbg["hidden"][b, 1], io["hidden"][i, 1])
        dl = abs(np.log(float(dbg["p"][b, 0])) - np.log(float(io["p"][i, 0])))
        assert dl <= bound, f"{name} b={b}: exit-head ln p error {dl:.3g} > bound {bound:.3g}"
        for l in (1, 2):
            k, v = k_gpu[(l, b)]
            kr = oc.K[l - 1, i, :, :P + 1].transpose(1, 0, 2)
            vr = oc.V[l - 1, i, :, :P + 1].transpose(1, 0, 2)
            assert maxrel(from_bf16_bits(k), kr) <= TOL and maxrel(from_bf16_bits(v), vr) <= TOL


def test_wide_passes_at_the_8b_widths_batch_64():
    """The batch-64 configuration's matrix-core (wide) passes at the 8B widths
    (d 4096, 32/8 heads of 128, F 14336, V 128256, int4 G128) on two layers:
    every projection and both vocabulary GEMVs see the full-size shapes.
    Sequences 0 and 63 against the oracle: at full depth (hidden states,
    logits, token, K/V), and with every row forced out after layer 1 (layer 2
    on the int4 copy through the wide int4 pass; the exit head's wide pass runs
    after layer 1 for all 64 rows)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_shared_exit_amd import api
    wl = synth.workload("8b_b64")
    sh = dataclasses.replace(wl.shape, n_layers=2)
    w = synth.make_weights(sh, wl.seed_weights)
    Bw, P = 64, 3
    prompts = np.random.default_rng(79).integers(0, sh.vocab, (Bw, P)).astype(np.int32)
    dev = api.upload_weights(w)
    out = {}
    split = np.array([1] * 32 + [0] * 32, np.int32)
    for label, gamma, forced in (("full", 2.0, None), ("exit1", 0.75, np.ones(Bw, np.int32)),
                                 ("split", 2.0, split)):
        model = api.Model(sh, dev, gamma=gamma, max_batch=Bw, max_positions=P + 2)
        cache = api.KVCache(model, Bw, P + 2, track=True)
        try:
            tg, lg = api.prefill(model, cache, prompts, logits=True)
            dbg = {"logits": None, "hidden": None, "p": None}
            t1, e1 = api.decode_step(model, cache, Bw, tokens=tg, forced=forced, debug=dbg)
            kv = {b: cache.read(2, b, 0, P + 1) for b in (0, 63)}
            assert np.all(cache.occupancy()[:, :Bw, :P + 1] == 1)
            out[label] = (tg, lg, t1, e1, dbg, kv)
        finally:
            cache.close()
            model.close()
    orc = om.OracleModel(sh, w, cache_f64=True)
    for b in (0, 63):
        for label in ("full", "exit1", "split"):
            tg, lg, t1, e1, dbg, kv = out[label]
            oc = om.KVCache(sh, 1, P + 2)
            to, info = om.prefill(orc, oc, prompts[b:b + 1])
            assert maxrel(lg[b], info["logits"][0]) <= TOL, f"{label} b={b} prefill logits"
            forced = None if label == "full" else [1] if label == "exit1" else [int(split[b])]
            t2, e2, io = om.decode_step(orc, oc, tg[b:b + 1], gamma=2.0 if label == "split" else 0.75,
                                        forced=forced, trace=True, heads=label != "full")
            assert e1[b] == e2[0]
            for l in range(sh.n_layers + 1):
                e = maxrel(dbg["hidden"][b, l], io["hidden"][0, l])
                assert e <= TOL, f"{label} b={b}: hidden after layer {l}: maxrel {e:.3g}"
            e = maxrel(dbg["logits"][b], io["logits"][0])
            assert e <= TOL, f"{label} b={b}: logits maxrel {e:.3g}"
            band = max(1e-2, 2 * float(np.abs(dbg["logits"][b].astype(np.float64) - io["logits"][0]).max()))
            if io["gap"][0] > band:
                assert t1[b] == t2[0], f"{label} b={b}: token"
            if label != "full":   # the exit head ran after layer 1 for every row (wide pass)
                bound = head_lnp_bound(orc, 1, dbg["hidden"][b, 1], io["hidden"][0, 1])
                dl = abs(np.log(float(dbg["p"][b, 0])) - np.log(float(io["p"][0, 0])))
                assert dl <= bound, f"{label} b={b}: exit-head ln p error {dl:.3g} > bound {bound:.3g}"
            k, v = kv[b]
            kr = oc.K[1, 0, :, :P + 1].transpose(1, 0, 2)
            vr = oc.V[1, 0, :, :P + 1].transpose(1, 0, 2)
            assert maxrel(from_bf16_bits(k), kr) <= TOL and maxrel(from_bf16_bits(v), vr) <= TOL, f"{label} KV"


def test_sampled_step_at_full_size(env):
    """Sampled decoding with AdaDecode's verification at the benchmark's shape
    (8B, batch 8, calibrated heads): sequence 0 forced out after layer 8 (its
    draft comes from the exit head there and is verified after the int4
    layers), sequence 1 at full depth (drawn from the final distribution);
    both tokens equal the oracle's wherever the draws are clear of rounding."""
    from parity import SAMPLE_BAND, ACCEPT_BAND
    api, w, dev = env
    P, tau = 2, 1.0
    prompts = _prompts(P)
    forced = np.array([8, SH.n_layers] + [12] * (B - 2), np.int32)
    model = api.Model(SH, dev, gamma=0.75, max_batch=B, max_positions=P + 2, temperature=tau, sample_seed=31)
    cache = api.KVCache(model, B, P + 2)
    try:
        tg = api.prefill(model, cache, prompts)
        dbg = {"logits": None, "p": None}
        t1, e1 = api.decode_step(model, cache, B, tokens=tg, forced=forced, debug=dbg)
        np.testing.assert_array_equal(e1, forced)
    finally:
        cache.close()
        model.close()
    # sequences 0 and 1 as a batch of two (a sequence's step does not depend on
    # the others in its batch)
    orc = om.OracleModel(SH, w, cache_f64=False)
    oc = om.KVCache(SH, 2, P + 2)
    om.prefill(orc, oc, prompts[:2])
    to, eo, io = om.decode_step(orc, oc, tg[:2], forced=forced[:2], temperature=tau, seed=31)
    compared = 0
    for b in (0, 1):
        assert eo[b] == forced[b]
        eps = float(np.abs(dbg["logits"][b].astype(np.float64) - io["logits"][b]).max())
        si = io["sample"][b]
        mg = si["margins"]
        gaps = [mg[0]] + mg[2:] if si["draft"] is not None else mg
        assert (si["draft"] is not None) == (b == 0)
        if min(gaps) > SAMPLE_BAND + 2 * eps / tau and (si["draft"] is None or mg[1] > ACCEPT_BAND):
            assert t1[b] == to[b], f"b={b}: sampled token gpu {t1[b]} oracle {to[b]} ({si})"
            compared += 1
    assert compared >= 1


@pytest.mark.parametrize("exit_after_1", [False, True], ids=["full", "exit1"])
def test_prefill_gemm_at_full_width(exit_after_1):
    """Two layers with the 8B widths (d 4096, 32/8 heads of 128, F 14336, V
    128256, G 128), batch 2, 520 prompt positions given as a 512-position call
    then an 8-position call (the second call's queries attend to the first's
    slots).  With exit_after_1 the sequence-level exit's threshold after layer
    1 is below any similarity, so both sequences leave and layer 2 runs the
    int4 copies in the GEMMs (in one call of all 520 positions, as the exit
    needs every token's similarity)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_shared_exit_amd import api, _binding as Bd
    from parity import GAP_BAND
    sh = dataclasses.replace(SH, n_layers=2)
    w = synth.make_weights(sh, 23)
    for lw in w["layers"]:
        lw.pop("head_T", None)
    Bp, P = 2, 520
    prompts = np.random.default_rng(80).integers(0, sh.vocab, (Bp, P)).astype(np.int32)
    dev = api.upload_weights(w)
    kw = dict(criterion=Bd.EE_CRIT_STS, gamma=-2.0 if exit_after_1 else 2.0, prefill_exit=exit_after_1)
    m = api.Model(sh, dev, max_batch=Bp, max_positions=P + 1, **kw)
    c = api.KVCache(m, Bp, P + 1, track=True)
    try:
        if exit_after_1:
            tg, lg, eg = api.prefill(m, c, prompts, logits=True, exits=True)
            np.testing.assert_array_equal(eg, [1, 1])
        else:
            api.prefill(m, c, prompts[:, :512])
            tg, lg = api.prefill(m, c, prompts[:, 512:], logits=True)
        assert np.all(c.occupancy()[:, :Bp, :P] == 1)
        pos = [0, 1, 255, 511, 512, 519]
        kv = {(l, b, p): c.read(l, b, p, 1) for l in (1, 2) for b in range(Bp) for p in pos}
    finally:
        c.close()
        m.close()
    orc = om.OracleModel(sh, w, cache_f64=True)
    oc = om.KVCache(sh, Bp, P + 1)
    to, info = om.prefill(orc, oc, prompts, exit_tau=-2.0 if exit_after_1 else None)
    if exit_after_1:
        np.testing.assert_array_equal(info["exit"], [1, 1])
    for b in range(Bp):
        e = maxrel(lg[b], info["logits"][b])
        print(f"b={b} last-position logits maxrel {e:.3g}", flush=True)
        assert e <= TOL, f"b={b} logits maxrel {e:.3g}"
        band = max(GAP_BAND, 2 * float(np.abs(lg[b].astype(np.float64) - info["logits"][b]).max()))
        if info["gap"][b] > band:
            assert tg[b] == to[b]
        for l in (1, 2):
            kg = np.concatenate([kv[(l, b, p)][0] for p in pos])
            vg = np.concatenate([kv[(l, b, p)][1] for p in pos])
            kr = oc.K[l - 1, b][:, pos].transpose(1, 0, 2)
            vr = oc.V[l - 1, b][:, pos].transpose(1, 0, 2)
            ek, ev = maxrel(from_bf16_bits(kg), kr), maxrel(from_bf16_bits(vg), vr)
            assert ek <= TOL and ev <= TOL, f"b={b} layer {l} K/V maxrel {ek:.3g} {ev:.3g}"
