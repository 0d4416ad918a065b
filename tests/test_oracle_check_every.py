"""Pins of evaluating the exit criterion only every N layers (CALM explainer,
"check every N layers"; AdaDecode's layer subsets): N = 1 is the default
step; N >= L evaluates nothing (the full-depth decoder); and checking every N
layers decides exactly like checking every layer with the thresholds of the
skipped layers raised above any reachable value (gamma 2: p <= 1, tau 2:
cos <= 1), for either criterion."""
import numpy as np
import pytest

import synth
from synth import ModelShape
from oracle import model as om

SH = ModelShape(5, 96, 6, 2, 16, 160, 300, 32, rope_theta=500000.0)


def _run(gamma, criterion="head", check_every=1, forced=None, steps=4, P=5, B=3, seed=21):
    w = synth.make_weights(SH, seed, alpha=np.full(SH.n_layers - 1, 40.0))
    m = om.OracleModel(SH, w)
    cache = om.KVCache(SH, B, P + steps + 1)
    tok, _ = om.prefill(m, cache, np.random.default_rng(3).integers(0, SH.vocab, (B, P)))
    out = []
    for _ in range(steps):
        tok, e, info = om.decode_step(m, cache, tok, gamma=gamma, forced=forced, criterion=criterion,
                                      check_every=check_every)
        out.append((tok.copy(), e.copy(), info["p"].copy()))
    return out, cache


def _gamma_with_skips(g, n, L):
    g = np.broadcast_to(np.asarray(g, np.float64), (L - 1,)).copy()
    for l in range(1, L):
        if l % n:
            g[l - 1] = 2.0
    return g


@pytest.mark.parametrize("criterion,gamma", [("head", 0.0040), ("sts", 0.77)])
@pytest.mark.parametrize("n", [2, 3])
def test_every_n_equals_raised_thresholds_between_checks(criterion, gamma, n):
    a, ca = _run(gamma, criterion, check_every=n)
    b, cb = _run(_gamma_with_skips(gamma, n, SH.n_layers), criterion)
    seen = set()
    for (ta, ea, pa), (tb, eb, pb) in zip(a, b):
        np.testing.assert_array_equal(ta, tb)
        np.testing.assert_array_equal(ea, eb)
        for l in range(1, SH.n_layers):
            col = pa[:, l - 1]
            if l % n:
                assert np.all(np.isnan(col)), "no criterion between checks"
            else:
                np.testing.assert_array_equal(col[np.isfinite(col)], pb[:, l - 1][np.isfinite(col)])
        seen.update(ea.tolist())
    assert all(e % n == 0 or e == SH.n_layers for e in seen)
    assert len(seen - {SH.n_layers}) > 0, "some sequence should exit at a check layer"
    np.testing.assert_array_equal(ca.K, cb.K)


def test_every_one_is_the_default():
    a, _ = _run(0.02, check_every=1)
    b, _ = _run(0.02)
    for (ta, ea, pa), (tb, eb, pb) in zip(a, b):
        np.testing.assert_array_equal(ta, tb)
        np.testing.assert_array_equal(ea, eb)
        np.testing.assert_array_equal(pa, pb)


def test_every_l_or_more_evaluates_nothing_and_is_full_depth():
    a, _ = _run(-1.0, check_every=SH.n_layers)
    b, _ = _run(2.0)
    for (ta, ea, pa), (tb, eb, _) in zip(a, b):
        assert np.all(ea == SH.n_layers) and np.all(np.isnan(pa))
        np.testing.assert_array_equal(ta, tb)


def test_forced_exits_apply_between_checks():
    a, _ = _run(2.0, check_every=3, forced=[1, 2, 4], steps=2)
    for _, ea, pa in a:
        np.testing.assert_array_equal(ea, [1, 2, 4])
        assert np.isnan(pa[0, 0]) and np.isnan(pa[1, 1])   # layers 1, 2: no criterion evaluated


def test_bad_check_every_is_refused():
    w = synth.make_weights(SH, 21)
    m = om.OracleModel(SH, w)
    cache = om.KVCache(SH, 1, 4)
    with pytest.raises(ValueError):
        om.decode_step(m, cache, [1], check_every=0)
