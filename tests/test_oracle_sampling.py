"""Pins of the oracle's sampled decoding with AdaDecode's verification
(AdaDecode explainer, section 3.1): the counter-based generator against
numpy's independent Philox4x64, the Gumbel-max draws against the softmax they
sample, the verified token's distribution against the final distribution (the
rejection-sampling identity) and the acceptance rate against its closed form
sum_t min(p_draft, p_final), and the low-temperature limit against greedy
decoding."""
import numpy as np
import pytest

import synth
from synth import ModelShape
from oracle import model as om
from oracle import sampling as sp

SH = ModelShape(3, 96, 6, 2, 16, 160, 300, 32, rope_theta=500000.0)
N = 20000  # draws per statistical check: every cell within 5 standard errors


def _within(freq, p, n=N):
    se = np.sqrt(p * (1 - p) / n)
    return np.all(np.abs(freq - p) <= 5 * se + 1e-12)


@pytest.mark.parametrize("counter,key", [((5, 7, 9, 11), (123, 456)), ((0, 0, 0, 1), (0, 0)),
                                         ((2**64 - 1, 3, 0, 2), (2**63, 17)),
                                         ((12345, 2, 999, 4), (2**64 - 1, 0))])
def test_philox_matches_numpy(counter, key):
    mine = [int(w) for w in sp.philox4x64([np.uint64(c) for c in counter], key)]
    c = sum(v << (64 * i) for i, v in enumerate(counter))
    k = key[0] + (key[1] << 64)
    # numpy advances the counter before each block: counter c - 1 yields block c
    ref = [int(x) for x in np.random.Philox(counter=(c - 1) % 2**256, key=k).random_raw(4)]
    assert mine == ref


def test_uniform_words_follow_block_layout():
    # word v % 4 of block v // 4, vectorised draw equal to single-block calls
    u = sp.uniforms(77, 5, 3, sp.STREAM_DRAFT, 10)
    for v in (0, 3, 4, 9):
        w = sp.philox4x64((np.uint64(v // 4), np.uint64(3), np.uint64(5), np.uint64(sp.STREAM_DRAFT)), (77, 0))
        x = int(w[v % 4])
        assert u[v] == ((x >> 41) + 0.5) * 2.0 ** -23
    assert np.all((u > 0) & (u < 1))
    np.testing.assert_array_equal(u.astype(np.float32).astype(np.float64), u)


def test_gumbel_max_draws_the_softmax():
    logits = np.array([1.0, -0.5, 0.3, 2.0, 0.0, -3.0])
    tau = 0.8
    p = sp.softmax_t(logits, tau)
    hits = np.zeros(len(logits))
    for pos in range(N):
        i, _ = sp.gumbel_argmax(logits / tau, sp.gumbel(9, pos, 1, sp.STREAM_FINAL, len(logits)))
        hits[i] += 1
    assert _within(hits / N, p)


def test_verified_token_follows_the_final_distribution():
    # draft and final distributions far apart: a missing min(1, .) or relu
    # correction, or drafting from the wrong distribution, shifts the result
    le = np.array([2.0, 0.0, -1.0, 1.5, -2.0])
    lf = np.array([-1.0, 1.0, 0.5, 0.0, 1.2])
    tau = 1.0
    pf, pd = sp.softmax_t(lf, tau), sp.softmax_t(le, tau)
    hits = np.zeros(len(lf))
    acc = 0
    for pos in range(N):
        t, info = sp.sample_token(lf, le, tau, 3, pos, 0)
        hits[t] += 1
        acc += info["accepted"]
    assert _within(hits / N, pf)
    assert not _within(hits / N, pd)
    alpha = np.minimum(pd, pf).sum()   # acceptance probability of the draft
    assert abs(acc / N - alpha) <= 5 * np.sqrt(alpha * (1 - alpha) / N)


def test_identical_distributions_always_accept():
    lf = np.array([0.1, 0.7, -0.2, 0.4])
    for pos in range(200):
        t, info = sp.sample_token(lf, lf.copy(), 0.9, 5, pos, 2)
        assert info["accepted"] and t == info["draft"]


def test_without_a_draft_the_final_distribution_is_sampled():
    lf = np.array([0.5, -0.5, 1.5, 0.0])
    pf = sp.softmax_t(lf, 1.3)
    hits = np.zeros(4)
    for pos in range(N):
        t, info = sp.sample_token(lf, None, 1.3, 11, pos, 7)
        assert info["draft"] is None
        hits[t] += 1
    assert _within(hits / N, pf)


def _run(temperature, steps=4, P=5, B=3, gamma=0.75, seed=21):
    w = synth.make_weights(SH, seed)
    m = om.OracleModel(SH, w)
    cache = om.KVCache(SH, B, P + steps + 1)
    tok, _ = om.prefill(m, cache, np.random.default_rng(3).integers(0, SH.vocab, (B, P)))
    out = []
    for s in range(steps):
        forced = np.array([1 + (b + s) % SH.n_layers for b in range(B)])  # drafts from every layer
        tok, e, info = om.decode_step(m, cache, tok, gamma=gamma, forced=forced, temperature=temperature, seed=4)
        out.append((tok.copy(), e.copy(), info))
    return out


def test_low_temperature_is_greedy_decoding():
    # tau -> 0: the draft is the exit head's argmax, accepted iff it is the
    # final argmax, and otherwise the residual is the final argmax's one-hot
    greedy = _run(0.0)
    cold = _run(1e-5)
    checked = 0
    for (tg, eg, ig), (tc, ec, ic) in zip(greedy, cold):
        np.testing.assert_array_equal(eg, ec)
        for b in range(len(tg)):
            if ig["gap"][b] > 1e-3:
                assert tc[b] == tg[b]
                checked += 1
        if tg[0] != tc[0]:
            break  # the greedy and sampled generations part ways from here
    assert checked >= 6


def test_sampled_step_records_decisions():
    out = _run(1.0)
    tok, e, info = out[0]
    for b, si in enumerate(info["sample"]):
        if e[b] < SH.n_layers:
            assert si["draft"] is not None and si["accepted"] in (True, False)
            if si["accepted"]:
                assert tok[b] == si["draft"]
        else:
            assert si["draft"] is None


def test_sampling_needs_the_exit_head_every_layer():
    w = synth.make_weights(SH, 21)
    m = om.OracleModel(SH, w)
    cache = om.KVCache(SH, 1, 4)
    with pytest.raises(ValueError):
        om.decode_step(m, cache, [1], criterion="sts", temperature=1.0)
    with pytest.raises(ValueError):
        om.decode_step(m, cache, [1], check_every=2, temperature=1.0)
