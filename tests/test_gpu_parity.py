"""GPU parity of the whole decode step against the oracle (runs through the C ABI)."""
import numpy as np
import pytest

import synth
from synth import ModelShape, Workload
from oracle.calibrate import calibrate

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny": synth.TINY,
    # widths that are not multiples of any tile, one kv head for five q heads,
    # int4 rows shorter than one 2048-element block, a ragged vocabulary
    "odd": ModelShape(3, 160, 5, 1, 32, 224, 1003, 32, rope_theta=500000.0),
    # full int4 blocks plus a tail (5120 = 2*2048 + 1024), an input wider than
    # the LDS-staged limit (down projection K = 5120), head_dim 128, 4 q per kv head
    "mid": ModelShape(3, 2048, 16, 4, 128, 5120, 5000, 128, rope_theta=500000.0),
    # head_dim 64 with 8 kv heads, group 64
    "hd64": ModelShape(2, 512, 8, 8, 64, 1024, 2048, 64, rope_theta=10000.0),
    # head_dim 64 with 4 q heads per kv head (the 1B attention), group 128
    "gqa4": ModelShape(3, 1024, 16, 4, 64, 2048, 2000, 128, rope_theta=500000.0),
}


def _weights(name, mean_exit, P, steps, gamma=0.75, seed=5):
    sh = SHAPES[name]
    wl = Workload(name, sh, 1, P, steps + 1, gamma, "calibrated", mean_exit, index=seed)
    cal = calibrate(wl, verbose=False)
    return sh, synth.make_weights(sh, seed, alpha=np.array(cal["alpha"]))


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_shared_exit_amd import _binding
    _binding.load()
    return torch


def test_tiny_workload_full_generation(gpu):
    from parity import run_parity
    wl = synth.workload("tiny")
    sh = wl.shape
    alpha = synth.load_alpha(wl)
    w = synth.make_weights(sh, wl.seed_weights, alpha=alpha)
    res = run_parity(sh, w, 1, wl.prompt_len, wl.decode_steps, wl.gamma,
                     prompts=synth.make_prompts(wl), label="tiny")
    assert res.compared_tokens >= 20


@pytest.mark.parametrize("name,batch,P,steps", [("tiny", 3, 9, 8), ("odd", 4, 7, 6),
                                                ("hd64", 5, 40, 4)])
def test_small_shapes_batched(gpu, name, batch, P, steps):
    from parity import run_parity
    sh = SHAPES[name]
    sh, w = _weights(name, min(2.0, sh.n_layers - 0.5), P, steps)
    res = run_parity(sh, w, batch, P, steps, 0.75, label=name)
    ex = np.stack(res.exits)
    assert ex.min() < sh.n_layers     # some exits happened


def test_mid_shape_long_context(gpu):
    """Contexts over several 256-position attention chunks plus a ragged tail."""
    from parity import run_parity
    sh, w = _weights("mid", 2.0, 16, 2)
    res = run_parity(sh, w, 3, 300, 3, 0.75, label="mid")


@pytest.mark.parametrize("name", ["odd", "mid"])
def test_forced_exit_schedule(gpu, name):
    """Per-sequence forced exits diverging inside the batch, every layer 1..L."""
    from parity import run_parity
    sh = SHAPES[name]
    w = synth.make_weights(sh, 9)
    L = sh.n_layers
    B = 6
    rng = np.random.default_rng(4)
    res = run_parity(sh, w, B, 5, 5, 0.75, forced_fn=lambda s: rng.integers(1, L + 1, B),
                     label=f"{name}-forced")


@pytest.mark.parametrize("name,batch", [("odd", 5), ("mid", 8)])
def test_every_row_exited_after_layer_one(gpu, name, batch):
    """Every sequence exits after layer 1, so layers 2..L run only exited rows:
    the projections take the smaller grid of that case (widths with int4 tails
    and ragged 16-row tiles in "odd", a 5120-column input in "mid")."""
    from parity import run_parity
    sh = SHAPES[name]
    w = synth.make_weights(sh, 13)
    res = run_parity(sh, w, batch, 5, 3, 0.75, forced_fn=lambda s: np.ones(batch, np.int32),
                     label=f"{name}-all-exited")
    for e in res.exits:
        assert (e == 1).all(), e


@pytest.mark.parametrize("name", ["odd", "mid"])
def test_unquantised_exit_copies(gpu, name):
    from parity import run_parity
    sh, w = _weights(name, 1.6, 6, 4)
    run_parity(sh, w, 3, 6, 4, 0.75, exit_mode="bf16", label=f"{name}-bf16")


def test_long_context_several_tiles_per_wave(gpu):
    """8 sequences x 8 kv heads x 2100 positions: each attention wave owns several
    64-position tiles (online softmax across tiles), plus a ragged last tile."""
    from parity import run_parity
    sh = SHAPES["hd64"]
    w = synth.make_weights(sh, 12)
    run_parity(sh, w, 8, 2100, 2, 0.75, forced_fn=lambda s: np.array([1, 2, 2, 1, 2, 2, 1, 2]),
               label="hd64-long", check_kv=False)


@pytest.mark.parametrize("name,batch", [("odd", 11), ("mid", 10)])
def test_more_than_eight_rows(gpu, name, batch):
    """More rows than one 8-row pass: the projections run the rows in chunks of 8
    (the later chunks read their ids from the lists), with forced exits so both
    weight formats have rows in every chunk."""
    from parity import run_parity
    sh = SHAPES[name]
    w = synth.make_weights(sh, 13)
    L = sh.n_layers
    rng = np.random.default_rng(8)
    res = run_parity(sh, w, batch, 4, 3, 0.75, forced_fn=lambda s: rng.integers(1, L + 1, batch),
                     label=f"{name}-b{batch}")
    ex = np.stack(res.exits)
    assert ex.min() < L and ex.max() == L


def test_gqa4_head_dim_64(gpu):
    from parity import run_parity
    sh, w = _weights("gqa4", 2.0, 20, 3)
    run_parity(sh, w, 4, 20, 3, 0.75, label="gqa4")


# ---------------------------------------------------------------------------
# River-LLM's state transition similarity as the exit criterion
# ---------------------------------------------------------------------------
def _median_similarity(sh, w, B, P, steps, seed):
    """Per-layer median of the oracle's similarity values at full depth (tau = 1:
    nobody exits) on prompts of another seed: thresholds that split the rows."""
    from oracle import model as om
    m = om.OracleModel(sh, w)
    c = om.KVCache(sh, B, P + steps + 1)
    tok, _ = om.prefill(m, c, np.random.default_rng(seed).integers(0, sh.vocab, (B, P)))
    vals = []
    for _ in range(steps):
        tok, _, info = om.decode_step(m, c, tok, gamma=1.0, criterion="sts")
        vals.append(info["p"])
    return np.median(np.concatenate(vals, axis=0), axis=0)


@pytest.mark.parametrize("name,batch,P,steps", [("tiny", 3, 9, 8), ("odd", 4, 7, 6), ("gqa4", 4, 12, 5)])
def test_similarity_criterion_against_oracle(gpu, name, batch, P, steps):
    from parity import run_parity
    sh = SHAPES[name]
    w = synth.make_weights(sh, 31)
    tau = _median_similarity(sh, w, batch, P, steps, seed=99)
    res = run_parity(sh, w, batch, P, steps, tau, criterion="sts", label=f"{name}-sts")
    exits = np.concatenate(res.exits)
    assert (exits < sh.n_layers).any() and (exits > 1).any(), "thresholds should split the rows"
    assert res.compared_tokens >= batch * steps // 2


def test_similarity_extremes_equal_the_head_extremes_bitwise(gpu):
    """tau = 1 (nobody exits) runs what the exit-head model runs at gamma = 2,
    and tau = -1.5 (everybody exits after layer 1) what it runs at gamma = -1:
    tokens, exit layers and K/V bitwise equal (the criterion only decides)."""
    from kv_shared_exit_amd import api, _binding as B
    sh = SHAPES["odd"]
    w = synth.make_weights(sh, 31)
    dev = api.upload_weights(w)
    P, steps, batch = 6, 5, 3
    prompts = np.random.default_rng(4).integers(0, sh.vocab, (batch, P)).astype(np.int32)

    def run(crit, g):
        m = api.Model(sh, dev, gamma=g, criterion=crit, max_batch=batch, max_positions=P + steps + 1)
        c = api.KVCache(m, batch, P + steps + 1)
        try:
            api.prefill(m, c, prompts)
            out = [api.decode_step(m, c, batch) for _ in range(steps)]
            kv = [c.read(l, b, 0, P + steps) for l in range(1, sh.n_layers + 1) for b in range(batch)]
        finally:
            c.close()
            m.close()
        return out, kv

    for (g_sts, g_head, e_all) in ((1.0, 2.0, sh.n_layers), (-1.5, -1.0, 1)):
        a, ka = run(B.EE_CRIT_STS, g_sts)
        b, kb = run(B.EE_CRIT_HEAD, g_head)
        for (ta, ea), (tb, eb) in zip(a, b):
            assert np.all(ea == e_all) and np.all(eb == e_all)
            np.testing.assert_array_equal(ta, tb)
        for (k1, v1), (k2, v2) in zip(ka, kb):
            np.testing.assert_array_equal(k1, k2)
            np.testing.assert_array_equal(v1, v2)


# ---------------------------------------------------------------------------
# The criterion evaluated only every N layers
# ---------------------------------------------------------------------------
FIVE = ModelShape(5, 256, 8, 2, 32, 512, 1500, 32, rope_theta=500000.0)


def test_check_every_two_layers_against_oracle(gpu):
    from parity import run_parity
    sh = FIVE
    w = synth.make_weights(sh, 41)
    tau = _median_similarity(sh, w, 3, 8, 5, seed=98)
    res = run_parity(sh, w, 3, 8, 5, tau, criterion="sts", check_every=2, label="five-sts-every2")
    exits = np.concatenate(res.exits)
    assert set(exits.tolist()) <= {2, 4, 5}
    assert (exits < sh.n_layers).any()


def test_check_every_equals_raised_thresholds_bitwise(gpu):
    """Checking every N layers decides like checking every layer with the
    thresholds of the layers in between raised to 2 (unreachable): tokens,
    exit layers and K/V bitwise equal, head criterion with forced exits mixed in."""
    from kv_shared_exit_amd import api, _binding as B
    sh = FIVE
    wl = Workload("five", sh, 1, 8, 6, 0.75, "calibrated", 2.5, index=7)
    cal = calibrate(wl, verbose=False)
    w = synth.make_weights(sh, 7, alpha=np.array(cal["alpha"]))
    dev = api.upload_weights(w)
    P, steps, batch, n = 8, 5, 4, 2
    prompts = np.random.default_rng(6).integers(0, sh.vocab, (batch, P)).astype(np.int32)
    g = np.full(sh.n_layers - 1, 0.75)
    g_raised = g.copy()
    g_raised[[l - 1 for l in range(1, sh.n_layers) if l % n]] = 2.0
    forced = np.array([0, 3, 0, 0], np.int32)

    def run(gamma, every):
        m = api.Model(sh, dev, gamma=gamma, check_every=every, max_batch=batch, max_positions=P + steps + 1)
        c = api.KVCache(m, batch, P + steps + 1)
        try:
            api.prefill(m, c, prompts)
            out = [api.decode_step(m, c, batch, forced=forced) for _ in range(steps)]
            kv = [c.read(l, b, 0, P + steps) for l in range(1, sh.n_layers + 1) for b in range(batch)]
        finally:
            c.close()
            m.close()
        return out, kv

    a, ka = run(g, n)
    b, kb = run(g_raised, 1)
    for (ta, ea), (tb, eb) in zip(a, b):
        np.testing.assert_array_equal(ea, eb)
        np.testing.assert_array_equal(ta, tb)
        assert ea[1] == 3   # forced between checks
    for (k1, v1), (k2, v2) in zip(ka, kb):
        np.testing.assert_array_equal(k1, k2)
        np.testing.assert_array_equal(v1, v2)


# ---------------------------------------------------------------------------
# Degenerate and maximal shapes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,sh,batch,gamma", [
    # one layer: no exit head anywhere, every exit layer is 1 = L
    ("one-layer", ModelShape(1, 64, 2, 1, 32, 96, 50, 32), 2, 0.75),
    # a vocabulary of one token: p = 1 > gamma after layer 1, token always 0, gap +inf
    ("one-token-vocab", ModelShape(2, 64, 2, 2, 32, 96, 1, 32), 3, 0.75),
])
def test_degenerate_shapes(gpu, name, sh, batch, gamma):
    from parity import run_parity
    w = synth.make_weights(sh, 3)
    res = run_parity(sh, w, batch, 4, 3, gamma, label=name)
    exits = np.concatenate(res.exits)
    assert np.all(exits == 1)
    assert res.compared_tokens == batch * 4


def test_largest_batch(gpu):
    """64 sequences (the largest batch): every kernel runs its rows in chunks of 8."""
    from parity import run_parity
    sh, w = _weights("tiny", 2.0, 6, 3)
    res = run_parity(sh, w, 64, 6, 3, 0.75, label="tiny-b64")
    exits = np.concatenate(res.exits)
    assert len(set(exits.tolist())) >= 2
    assert res.compared_tokens >= 64 * 3


@pytest.mark.parametrize("label,sh,batch", [
    # 2 batch blocks of 16 (ragged), head_dim 64, group 64
    ("wide-hd64", SHAPES["hd64"], 24),
    # a vocabulary that ends inside a 16-row tile (1003), 3 batch blocks
    ("wide-odd-vocab", ModelShape(3, 256, 4, 2, 64, 512, 1003, 32, rope_theta=500000.0), 40),
    # every row of the largest batch (4 blocks of 16); F = 384 is not a multiple
    # of 256, so the projections keep the 8-row passes (vocabulary pass only)
    ("wide-b64", ModelShape(2, 256, 4, 2, 64, 384, 700, 32, rope_theta=10000.0), 64),
    # group 128, head_dim 128, one batch block plus one row
    ("wide-g128", ModelShape(3, 512, 4, 2, 128, 768, 500, 128, rope_theta=500000.0), 17),
    # group 128 with 3 and 4 batch blocks (the loop bodies specialised for
    # them), the rows of a layer split between the two formats
    ("wide-g128-b40", ModelShape(3, 512, 4, 2, 128, 768, 500, 128, rope_theta=500000.0), 40),
    ("wide-g128-b64", ModelShape(3, 512, 4, 2, 128, 768, 500, 128, rope_theta=500000.0), 64),
])
def test_wide_batch_vocabulary_pass(gpu, label, sh, batch):
    """Batches of more than 8 rows: the projections run on the matrix-core pass
    (both weight formats, column ranges summed by the epilogues) when the widths
    are multiples of 256; the exit head's vocabulary pass and the LM head run on
    the matrix-core pass over the tiled copy of E for any number of rows on the
    backbone; exits are spread so that some layers have more than 8 rows on the
    backbone and some fewer (the pass computes four 16-row batch blocks and
    keeps only the listed rows)."""
    from parity import run_parity
    wl = Workload(label, sh, 1, 6, 4, 0.75, "calibrated", max(1.2, sh.n_layers / 2), index=9)
    cal = calibrate(wl, verbose=False)
    w = synth.make_weights(sh, 9, alpha=np.array(cal["alpha"]))
    res = run_parity(sh, w, batch, 6, 3, 0.75, label=label)
    exits = np.concatenate(res.exits)
    assert len(set(exits.tolist())) >= 2
    assert res.compared_tokens >= batch * 2


def test_wide_vocabulary_pass_with_few_rows_on_the_backbone(gpu):
    """A step of 12 rows (the matrix-core passes) where 9 rows are forced out
    after layer 1: the exit head of layer 2 has 3 rows on the backbone and runs
    on the wide vocabulary pass, which serves every exit head of a step above
    8 rows; its p values (compared at every evaluated head) and the exits
    match the oracle."""
    from parity import run_parity
    sh = ModelShape(3, 512, 4, 2, 128, 768, 500, 128, rope_theta=500000.0)
    w = synth.make_weights(sh, 9)
    B = 12
    forced = np.where(np.arange(B) < 9, 1, 0).astype(np.int32)
    res = run_parity(sh, w, B, 6, 3, 2.0, forced_fn=lambda s: forced, label="wide-few-rows")
    assert res.compared_tokens >= B * 2
    exits = np.concatenate(res.exits)
    assert (exits == 1).sum() >= 9 and (exits == 3).sum() >= 3


def test_attention_one_workgroup_per_sequence_and_kv_head(gpu):
    """32 sequences x 8 kv heads (256 pairs): decode attention runs one
    workgroup per (sequence, kv head), whose 8 waves take the 9 tiles of each
    521..523-position context in turn (wave 0 two, the last tile ragged), and
    merges the waves' partial softmax states in LDS; half the rows exit after
    layer 1, so layer 2 runs both weight formats."""
    from parity import run_parity
    sh = SHAPES["hd64"]
    w = synth.make_weights(sh, 9)
    B = 32
    forced = np.where(np.arange(B) % 2 == 0, 1, 0).astype(np.int32)
    res = run_parity(sh, w, B, 520, 3, 2.0, forced_fn=lambda s: forced, label="fused-attn-b32")
    assert res.compared_tokens >= B * 2


# ---------------------------------------------------------------------------
# The batch-minimum exit rule
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("criterion", ["sts", "head"])
def test_batch_minimum_rule_against_oracle(gpu, criterion):
    from parity import run_parity
    sh = FIVE
    if criterion == "sts":
        w = synth.make_weights(sh, 41)
        # thresholds a little under the medians: the batch minimum crosses them now and then
        thr = _median_similarity(sh, w, 4, 8, 5, seed=98) - 0.05
    else:
        wl = Workload("five", sh, 1, 8, 6, 0.75, "calibrated", 1.5, index=7)
        w = synth.make_weights(sh, 7, alpha=np.array(calibrate(wl, verbose=False)["alpha"]))
        thr = 0.75
    res = run_parity(sh, w, 4, 8, 6, thr, criterion=criterion, exit_rule="batch_min",
                     label=f"five-{criterion}-batchmin")
    for e in res.exits:
        assert len(set(e.tolist())) == 1, f"one exit layer per step: {e}"
    assert any(e[0] < sh.n_layers for e in res.exits), "the batch should exit early in some step"


def test_batch_minimum_of_one_sequence_is_the_per_sequence_rule(gpu):
    from kv_shared_exit_amd import api, _binding as B
    sh = FIVE
    w = synth.make_weights(sh, 41)
    tau = _median_similarity(sh, w, 1, 8, 5, seed=97)
    dev = api.upload_weights(w)
    prompts = np.random.default_rng(8).integers(0, sh.vocab, (1, 8)).astype(np.int32)

    def run(rule):
        m = api.Model(sh, dev, gamma=tau, criterion=B.EE_CRIT_STS, exit_rule=rule, max_batch=1,
                      max_positions=16)
        c = api.KVCache(m, 1, 16)
        try:
            api.prefill(m, c, prompts)
            return [api.decode_step(m, c, 1) for _ in range(6)]
        finally:
            c.close()
            m.close()

    for (ta, ea), (tb, eb) in zip(run(B.EE_RULE_SEQUENCE), run(B.EE_RULE_BATCH_MIN)):
        np.testing.assert_array_equal(ea, eb)
        np.testing.assert_array_equal(ta, tb)


# ---------------------------------------------------------------------------
# Sampled decoding with AdaDecode's verification
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,batch,temperature", [("tiny", 4, 1.0), ("odd", 5, 0.7), ("hd64", 3, 1.5)])
def test_sampled_decoding_against_oracle(gpu, name, batch, temperature):
    """Draft at the exit layer (Gumbel-max of the exit head's logits / tau over
    Philox noise), acceptance with min(1, p_final / p_draft), resampling from
    relu(p_final - p_draft), and undrafted rows from p_final: tokens equal the
    oracle's wherever every draw and the acceptance test are clear of rounding.
    Forced exits spread the drafts over every layer (and leave some rows at
    full depth, which draw from the final distribution)."""
    from parity import run_parity
    sh, w = _weights(name, min(2.0, SHAPES[name].n_layers - 0.5), 7, 6)
    L = sh.n_layers
    forced = lambda s: np.array([1 + (b + s) % L for b in range(batch)], np.int32)
    res = run_parity(sh, w, batch, 7, 6, 0.75, forced_fn=forced, label=f"{name}-sampled",
                     temperature=temperature, seed=1234)
    outcomes = set(res.sample_outcomes)
    assert res.compared_tokens >= batch * 4
    assert "none" in outcomes and outcomes & {"accepted", "rejected"}, outcomes


def test_sampled_decoding_rejections_are_resampled(gpu):
    """Exit heads scaled up (alpha 3000: nearly one-hot exit distributions, so
    every row exits after layer 1 on its own criterion and the draft's
    probability is ~1): a draft is accepted only with the final distribution's
    probability of it, so most are rejected and the resampling pass decides
    most tokens."""
    from parity import run_parity
    sh = SHAPES["odd"]
    w = synth.make_weights(sh, 5, alpha=np.full(sh.n_layers - 1, 3000.0))
    res = run_parity(sh, w, 4, 6, 6, 0.75, label="odd-sampled-rejections", temperature=1.0, seed=99)
    assert res.sample_outcomes.count("rejected") >= 3, res.sample_outcomes


@pytest.mark.parametrize("batch,alpha", [(12, 7.0), (40, 3000.0)], ids=["b12", "b40-rejections"])
def test_sampled_decoding_above_8_rows(gpu, batch, alpha):
    """Sampled decoding on batches above 8 rows (a model with the matrix-core
    passes): the sampled vocabulary passes take the rows 8 at a time.  At 40
    rows with one-hot-like exit heads most drafts are rejected, so the
    resampling pass's list holds more than 32 row pairs."""
    from parity import run_parity
    sh = SHAPES["hd64"]   # widths of 256 multiples: the matrix-core passes run the other projections
    w = synth.make_weights(sh, 9, alpha=np.full(sh.n_layers - 1, alpha))
    L = sh.n_layers
    forced = (lambda s: np.array([1 + (b + s) % L for b in range(batch)], np.int32)) if alpha < 100 else None
    res = run_parity(sh, w, batch, 5, 3, 0.75, forced_fn=forced, label=f"sampled-b{batch}",
                     temperature=1.0, seed=77)
    assert res.compared_tokens >= batch
    if alpha > 100:
        assert res.sample_outcomes.count("rejected") >= 33, res.sample_outcomes.count("rejected")


def test_sampled_low_temperature_equals_greedy(gpu):
    """tau -> 0: the verified draw is the greedy token (the draft is the exit
    head's argmax, accepted iff it is the final argmax, else the residual's
    mass sits on the final argmax)."""
    from kv_shared_exit_amd import api
    sh, w = _weights("tiny", 2.0, 8, 5)
    dev = api.upload_weights(w)
    prompts = np.random.default_rng(8).integers(0, sh.vocab, (4, 8)).astype(np.int32)
    toks = {}
    for tau in (0.0, 1e-5):
        m = api.Model(sh, dev, gamma=0.75, max_batch=4, max_positions=16, temperature=tau, sample_seed=3)
        c = api.KVCache(m, 4, 16)
        t = api.prefill(m, c, prompts)
        seq = []
        for s in range(5):
            forced = np.array([1 + (b + s) % sh.n_layers for b in range(4)], np.int32)
            dbg = {"gap": None}
            t, e = api.decode_step(m, c, 4, tokens=t, forced=forced, debug=dbg)
            seq.append((t.copy(), dbg["gap"].copy()))
        toks[tau] = seq
        c.close()
        m.close()
    checked = 0
    for (tg, gap), (tc, _) in zip(toks[0.0], toks[1e-5]):
        for b in range(4):
            if gap[b] > 1e-3:
                assert tc[b] == tg[b]
                checked += 1
        if not np.array_equal(tg, tc):
            break
    assert checked >= 4


# ---------------------------------------------------------------------------
# River-LLM's sequence-level exit in the prefill
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,batch,P", [("odd", 3, 9), ("hd64", 4, 40), ("tiny", 2, 70)])
def test_prefill_sequence_exit_against_oracle(gpu, name, batch, P):
    """The prefill runs layer by layer; after layer l a sequence leaves when the
    smallest similarity of its prompt's tokens exceeds tau_l, and its later
    layers run on the int4 copies for every token.  Thresholds are placed
    between the sequences' token minima of the oracle's full-depth prefill
    (each at least 1e-3 away from every minimum), at a different layer per
    sequence where possible; exit layers equal the oracle's, and the last
    position's logits, the token and every K/V slot match it."""
    from kv_shared_exit_amd import api, _binding as Bd
    from parity import maxrel, TOL
    from oracle import model as om
    from oracle.numerics import from_bf16_bits
    sh = SHAPES[name]
    L = sh.n_layers
    w = synth.make_weights(sh, 13)
    prompts = np.random.default_rng(31).integers(0, sh.vocab, (batch, P)).astype(np.int32)
    orc = om.OracleModel(sh, w)
    oc = om.KVCache(sh, batch, P + 1)
    _, full = om.prefill(orc, oc, prompts, trace=True)
    hid = full["hidden"]                      # [B, P, L+1, d]
    mins = np.stack([om.state_transition_similarity(hid[:, :, l - 1], hid[:, :, l]).min(axis=1)
                     for l in range(1, L)], axis=1)   # [B, L-1]
    tau = np.full(L - 1, 2.0)
    for l in range(1, L):                     # the first layer whose minima split the batch
        v = np.sort(mins[:, l - 1])
        gaps = np.diff(v)
        if len(gaps) and gaps.max() > 2e-3:
            k = int(np.argmax(gaps))
            tau[l - 1] = 0.5 * (v[k] + v[k + 1])
            break
    assert np.all(np.abs(mins - tau[None, :]) > 1e-3)
    oc = om.KVCache(sh, batch, P + 1)
    to, info = om.prefill(orc, oc, prompts, exit_tau=tau)
    assert len(set(info["exit"].tolist())) >= 2, info["exit"]
    dev = api.upload_weights(w)
    m = api.Model(sh, dev, gamma=tau, max_batch=batch, max_positions=P + 1, criterion=Bd.EE_CRIT_STS,
                  prefill_exit=True)
    c = api.KVCache(m, batch, P + 1, track=True)
    try:
        tg, lg, eg = api.prefill(m, c, prompts, logits=True, exits=True)
        np.testing.assert_array_equal(eg, info["exit"])
        for b in range(batch):
            assert maxrel(lg[b], info["logits"][b]) <= TOL
            band = max(1e-2, 2 * float(np.abs(lg[b].astype(np.float64) - info["logits"][b]).max()))
            if info["gap"][b] > band:
                assert tg[b] == to[b]
            for l in range(1, L + 1):
                k, v = c.read(l, b, 0, P)
                kr = oc.K[l - 1, b, :, :P].transpose(1, 0, 2)
                vr = oc.V[l - 1, b, :, :P].transpose(1, 0, 2)
                assert maxrel(from_bf16_bits(k), kr) <= TOL and maxrel(from_bf16_bits(v), vr) <= TOL, (b, l)
        assert np.all(c.occupancy()[:, :batch, :P] == 1)
        assert list(c.lengths()[:batch]) == [P] * batch
        # decoding continues from the prefill's cache and token
        t1, e1 = api.decode_step(m, c, batch)
        assert np.all((e1 >= 1) & (e1 <= L))
    finally:
        c.close()
        m.close()


def test_prefill_exit_off_and_unreachable_thresholds_equal_full_depth(gpu):
    """prefill_exit with thresholds a similarity cannot exceed runs every layer on
    the backbone: it equals the prefill without the exit (tokens, exit layers,
    logits within rounding, K/V)."""
    from kv_shared_exit_amd import api, _binding as Bd
    from parity import maxrel, TOL
    from oracle.numerics import from_bf16_bits
    sh = SHAPES["odd"]
    w = synth.make_weights(sh, 14)
    dev = api.upload_weights(w)
    prompts = np.random.default_rng(2).integers(0, sh.vocab, (3, 12)).astype(np.int32)
    out = []
    for pe in (False, True):
        m = api.Model(sh, dev, gamma=1.0, max_batch=3, max_positions=13, criterion=Bd.EE_CRIT_STS, prefill_exit=pe)
        c = api.KVCache(m, 3, 13)
        try:
            t, lg, e = api.prefill(m, c, prompts, logits=True, exits=True)
            kv = [c.read(l, b, 0, 12) for l in (1, sh.n_layers) for b in range(3)]
            out.append((t, lg, e, kv))
        finally:
            c.close()
            m.close()
    (t0, l0, e0, kv0), (t1, l1, e1, kv1) = out
    assert np.all(e0 == sh.n_layers) and np.all(e1 == sh.n_layers)
    np.testing.assert_array_equal(t0, t1)
    for b in range(3):
        assert maxrel(l1[b], l0[b]) <= 1e-5
    for (k0, v0), (k1, v1) in zip(kv0, kv1):
        assert maxrel(from_bf16_bits(k1), from_bf16_bits(k0)) <= 1e-2


@pytest.mark.parametrize("name,batch,chunks", [("odd", 3, (20, 1, 24)), ("hd64", 2, (33, 31)),
                                               ("gqa4", 4, (64, 70))])
def test_prefill_in_chunks_against_oracle(gpu, name, batch, chunks):
    """The prefill's matrix-core path over several calls: each call appends its
    positions after the cached ones, so its queries attend to the earlier
    calls' K/V slots as well as to its own.  Against the oracle's prefill of
    the whole prompt: every K/V slot of every layer, the last position's
    logits and the token."""
    from kv_shared_exit_amd import api
    from parity import maxrel, TOL, GAP_BAND
    from oracle import model as om
    from oracle.numerics import from_bf16_bits
    sh = SHAPES[name]
    P = sum(chunks)
    w = synth.make_weights(sh, 15)
    prompts = np.random.default_rng(41).integers(0, sh.vocab, (batch, P)).astype(np.int32)
    dev = api.upload_weights(w)
    m = api.Model(sh, dev, gamma=2.0, max_batch=batch, max_positions=P + 1)
    c = api.KVCache(m, batch, P + 1, track=True)
    try:
        p0 = 0
        for n in chunks:
            tg, lg = api.prefill(m, c, prompts[:, p0:p0 + n], logits=True)
            p0 += n
        assert list(c.lengths()) == [P] * batch
        occ = c.occupancy()
        assert np.all(occ[:, :batch, :P] == 1) and np.all(occ[:, :batch, P:] == 0)
        kv = {(l, b): c.read(l, b, 0, P) for l in range(1, sh.n_layers + 1) for b in range(batch)}
    finally:
        c.close()
        m.close()
    orc = om.OracleModel(sh, w)
    oc = om.KVCache(sh, batch, P + 1)
    to, info = om.prefill(orc, oc, prompts)
    for b in range(batch):
        e = maxrel(lg[b], info["logits"][b])
        assert e <= TOL, f"{name} b={b} logits maxrel {e:.3g}"
        band = max(GAP_BAND, 2 * float(np.abs(lg[b].astype(np.float64) - info["logits"][b]).max()))
        if info["gap"][b] > band:
            assert tg[b] == to[b], f"{name} b={b} token"
        for l in range(1, sh.n_layers + 1):
            k, v = kv[(l, b)]
            kr = oc.K[l - 1, b, :, :P].transpose(1, 0, 2)
            vr = oc.V[l - 1, b, :, :P].transpose(1, 0, 2)
            ek, ev = maxrel(from_bf16_bits(k), kr), maxrel(from_bf16_bits(v), vr)
            assert ek <= TOL and ev <= TOL, f"{name} KV layer {l} seq {b}: {ek:.3g} {ev:.3g}"
