"""Pins of the oracle's state-transition-similarity exit criterion (River-LLM
explainer, sections 5.1-5.2): the similarity against closed forms and torch's
library normalisation, and the whole step at thresholds where the criterion's
outcome is fixed by the range of a cosine (tau >= 1: nobody exits; tau < -1:
everybody exits after layer 1), which reduce to cases pinned elsewhere."""
import numpy as np
import pytest
import torch

import synth
from synth import ModelShape
from oracle import model as om

SH = ModelShape(3, 96, 6, 2, 16, 160, 300, 32, rope_theta=500000.0)


def test_similarity_closed_forms():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((5, 33))
    np.testing.assert_allclose(om.state_transition_similarity(a, a), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(om.state_transition_similarity(a, -a), -1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(om.state_transition_similarity(a, 3.5 * a), 1.0, rtol=0, atol=1e-15)
    # orthogonal rows
    e1, e2 = np.eye(4)[:1], np.eye(4)[1:2]
    assert om.state_transition_similarity(e1, e2)[0] == 0.0
    # (1, 0) against (1, 1): cos 45 degrees
    np.testing.assert_allclose(om.state_transition_similarity([[1.0, 0.0]], [[1.0, 1.0]]), [2 ** -0.5],
                               rtol=1e-15)
    # scale invariance of either argument
    b = rng.standard_normal((5, 33))
    np.testing.assert_allclose(om.state_transition_similarity(7 * a, 0.25 * b),
                               om.state_transition_similarity(a, b), rtol=1e-13)


def test_similarity_matches_torch_normalize():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((7, 128)) * 0.02
    b = a + rng.standard_normal((7, 128)) * 0.01
    ta, tb = torch.from_numpy(a), torch.from_numpy(b)
    ref = (torch.nn.functional.normalize(ta, dim=-1) * torch.nn.functional.normalize(tb, dim=-1)).sum(-1)
    np.testing.assert_allclose(om.state_transition_similarity(a, b), ref.numpy(), rtol=1e-13, atol=1e-15)


def _run(criterion, gamma, steps=4, P=5, B=2, trace=False):
    w = synth.make_weights(SH, 21)
    m = om.OracleModel(SH, w)
    cache = om.KVCache(SH, B, P + steps + 1)
    prompts = np.random.default_rng(3).integers(0, SH.vocab, (B, P))
    tok, _ = om.prefill(m, cache, prompts)
    out = []
    for _ in range(steps):
        tok, e, info = om.decode_step(m, cache, tok, gamma=gamma, criterion=criterion, trace=trace)
        out.append((tok.copy(), e.copy(), info))
    return out, cache


def test_tau_at_least_one_never_exits_and_is_full_depth():
    sts, _ = _run("sts", 1.0, trace=True)
    full, _ = _run("head", 2.0)
    for (ts, es, infs), (tf, ef, inff) in zip(sts, full):
        assert np.all(es == SH.n_layers)
        np.testing.assert_array_equal(ts, tf)
        np.testing.assert_allclose(infs["logits"], inff["logits"], rtol=0, atol=0)
        # the recorded value of layer l is the cosine of the states before and after it
        hid = infs["hidden"]
        for l in range(1, SH.n_layers):
            a, b = torch.from_numpy(hid[:, l - 1]), torch.from_numpy(hid[:, l])
            ref = (torch.nn.functional.normalize(a, dim=-1) * torch.nn.functional.normalize(b, dim=-1)).sum(-1)
            np.testing.assert_allclose(infs["p"][:, l - 1], ref.numpy(), rtol=1e-12)
            assert np.all(infs["p"][:, l - 1] <= 1.0)


def test_tau_below_minus_one_exits_after_layer_one_like_the_head_at_gamma_zero():
    sts, c1 = _run("sts", -1.5)
    head, c2 = _run("head", -1.0)
    for (ts, es, _), (th, eh, _) in zip(sts, head):
        assert np.all(es == 1) and np.all(eh == 1)
        np.testing.assert_array_equal(ts, th)
    np.testing.assert_array_equal(c1.K, c2.K)
    np.testing.assert_array_equal(c1.V, c2.V)


def test_forced_exit_overrides_the_similarity():
    w = synth.make_weights(SH, 21)
    m = om.OracleModel(SH, w)
    cache = om.KVCache(SH, 2, 8)
    tok, _ = om.prefill(m, cache, np.random.default_rng(3).integers(0, SH.vocab, (2, 5)))
    # tau = -1.5 alone would exit both after layer 1
    _, e, info = om.decode_step(m, cache, tok, gamma=-1.5, forced=[1, 3], criterion="sts")
    np.testing.assert_array_equal(e, [1, 3])
    assert np.isfinite(info["p"][0, 0]) and np.isnan(info["p"][0, 1])   # not evaluated after its exit
    assert np.all(np.isfinite(info["p"][1]))


def test_unknown_criterion_is_refused():
    w = synth.make_weights(SH, 21)
    m = om.OracleModel(SH, w)
    cache = om.KVCache(SH, 1, 4)
    with pytest.raises(ValueError):
        om.decode_step(m, cache, [1], criterion="cosine")
