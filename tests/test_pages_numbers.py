"""The pages' printed numbers against the shapes and input recipe used here (CPU)."""
import json
import os

import numpy as np

import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_head_parameter_counts():
    g = GOLD["head_params"]
    d = synth.LLAMA8B.d_model
    assert d == g["d"]
    t_params = d * d                                # T is d x d
    assert abs(t_params - g["t_params"]) / g["t_params"] < 1e-3
    e_params = g["vocab_k"] * d
    assert abs(e_params - g["e_params"]) / g["e_params"] < 1e-3
    assert round(e_params / t_params) == g["ratio"]


def test_int4_copy_size():
    g = GOLD["int4_reduction"]
    sh = synth.LLAMA8B
    n = sh.params_per_layer()
    int4 = n / 2 + 2 * n / sh.group
    assert abs((1 - int4 / (2 * n)) - g["reduction"]) < g["tolerance"]


def test_exit_potential_and_target_distribution():
    g = GOLD["exit_potential"]
    assert abs(1 - g["mean_exit"] / g["layers"] - g["compute_cut"]) < 0.005
    assert abs(g["layers"] / g["mean_exit"] - g["speedup"]) < 0.05
    # the 1B workload's target exit distribution has the page's mean
    wl = synth.workload("1b")
    h = synth.geometric_hazard(wl.mean_exit, wl.shape.n_layers)
    pmf = synth.exit_pmf(h, wl.shape.n_layers)
    assert abs(pmf.sum() - 1) < 1e-12
    assert abs((pmf * np.arange(1, 17)).sum() - g["mean_exit"]) < 1e-9


def test_default_gamma():
    assert synth.workload("8b").gamma == GOLD["gamma_default"]["gamma"]


def test_target_exit_draws_follow_the_target_distribution():
    # the 1B page's mean exit layer (4.81 of 16); draws stand in for calibrated
    # heads where none exist, so their histogram must match the pmf
    wl = synth.workload("1b")
    L = wl.shape.n_layers
    e = np.concatenate([synth.make_target_exits(wl, s, batch=64) for s in range(500)])
    assert e.min() >= 1 and e.max() <= L
    pmf = synth.exit_pmf(synth.geometric_hazard(wl.mean_exit, L), L)
    freq = np.bincount(e, minlength=L + 1)[1:] / e.size
    # 32000 draws: every cell within 5 standard errors
    se = np.sqrt(pmf * (1 - pmf) / e.size)
    assert np.all(np.abs(freq - pmf) <= 5 * se + 1e-12)
    assert abs(e.mean() - g_mean(wl)) < 0.1
    # seeded: the same step gives the same draw, another step another
    np.testing.assert_array_equal(synth.make_target_exits(wl, 7, batch=8), synth.make_target_exits(wl, 7, batch=8))
    assert not np.array_equal(synth.make_target_exits(wl, 7, batch=64), synth.make_target_exits(wl, 8, batch=64))


def g_mean(wl):
    return GOLD["exit_potential"]["mean_exit"] if wl.name == "1b" else wl.mean_exit
