"""Pins of the batch-minimum exit rule (River-LLM explainer, section 5.2: the
exit fires when the minimum over the batch's tokens exceeds the threshold).
Until the batch exits every sequence runs the same layers as at full depth,
so the exit layer is fixed by a full-depth run: the first evaluated layer at
which the smallest value over the batch exceeds the threshold.  A batch of
one is the per-sequence rule; forced sequences keep their own layers and do
not take part in the minimum."""
import copy

import numpy as np
import pytest

import synth
from synth import ModelShape
from oracle import model as om

SH = ModelShape(5, 96, 6, 2, 16, 160, 300, 32, rope_theta=500000.0)


def _setup(B, P=5, steps=4, seed=21):
    w = synth.make_weights(SH, seed, alpha=np.full(SH.n_layers - 1, 40.0))
    m = om.OracleModel(SH, w)
    cache = om.KVCache(SH, B, P + steps + 1)
    tok, _ = om.prefill(m, cache, np.random.default_rng(3).integers(0, SH.vocab, (B, P)))
    return m, cache, tok


@pytest.mark.parametrize("criterion,tau", [("sts", 0.74), ("head", 0.0038)])
def test_exit_layer_follows_from_the_full_depth_values(criterion, tau):
    B = 4
    m, c, tok = _setup(B)
    layers = []
    for _ in range(4):
        # full depth from a copy of the same cache state: every layer's values
        _, _, full = om.decode_step(m, copy.deepcopy(c), tok, gamma=2.0, criterion=criterion)
        vals = full["p"]                                           # [B, L-1]
        above = [l for l in range(1, SH.n_layers) if vals[:, l - 1].min() > tau]
        expect = above[0] if above else SH.n_layers
        tok, e, info = om.decode_step(m, c, tok, gamma=tau, criterion=criterion, exit_rule="batch_min")
        assert np.all(e == expect)
        np.testing.assert_array_equal(info["p"][:, :expect], vals[:, :expect])
        assert np.all(np.isnan(info["p"][:, expect:]))
        layers.append(expect)
    assert len(set(layers) - {SH.n_layers}) >= 1, "the batch should exit early in some step"


def test_batch_of_one_is_the_per_sequence_rule():
    m1, c1, tok = _setup(1)
    m2, c2, _ = _setup(1)
    for _ in range(4):
        ta, ea, _ = om.decode_step(m1, c1, tok, gamma=0.74, criterion="sts")
        tb, eb, _ = om.decode_step(m2, c2, tok, gamma=0.74, criterion="sts", exit_rule="batch_min")
        np.testing.assert_array_equal(ea, eb)
        np.testing.assert_array_equal(ta, tb)
        tok = ta


def test_forced_sequences_keep_their_layers_and_leave_the_minimum():
    B = 3
    m, c, tok = _setup(B)
    # tau below every reachable value: the free sequences leave after layer 1
    t, e, _ = om.decode_step(m, c, tok, gamma=-1.5, criterion="sts", exit_rule="batch_min", forced=[0, 4, 0])
    np.testing.assert_array_equal(e, [1, 4, 1])


def test_unknown_rule_is_refused():
    m, c, tok = _setup(1)
    with pytest.raises(ValueError):
        om.decode_step(m, c, tok, exit_rule="majority")
