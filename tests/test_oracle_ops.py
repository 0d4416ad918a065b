"""Pins of the oracle's elementary operations against torch CPU routines and closed forms."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.numerics import bf16_round
from oracle import model as om


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((5, 96)) * 3
    g = bf16_round(rng.standard_normal(96))
    got = om.rmsnorm(h, g, 1e-5)
    ref = F.rms_norm(torch.from_numpy(h), (96,), weight=torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(got, bf16_round(ref), rtol=0, atol=0)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(om.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-15, atol=1e-300)


def test_rope_closed_form_value():
    """pos = 1, frequency index 0 (theta^0 = 1): (1, 0) turns into (cos 1, sin 1)."""
    cos, sin = om.rope_table(4, 8, 10000.0)
    x = np.zeros(8)
    x[0] = 1.0
    y = om.apply_rope(x, cos[1], sin[1])
    assert y[0] == bf16_round(np.float32(math.cos(1.0)))
    assert y[4] == bf16_round(np.float32(math.sin(1.0)))
    # pos 0 is the identity
    z = bf16_round(np.random.default_rng(0).standard_normal(8))
    np.testing.assert_array_equal(om.apply_rope(z, cos[0], sin[0]), z)
    # frequency i uses theta^(-2i/hd)
    assert cos[3, 1] == np.float32(math.cos(3 * 10000.0 ** (-2 / 8)))


def test_rope_relative_position_invariant():
    """Rotated dot products depend only on the position difference (before bf16 rounding)."""
    hd = 64
    cos, sin = om.rope_table(64, hd, 500000.0)
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)

    def rot(x, p):
        half = hd // 2
        x1, x2 = x[:half], x[half:]
        c, s = np.cos(p * 500000.0 ** (-np.arange(half) * 2 / hd)), np.sin(p * 500000.0 ** (-np.arange(half) * 2 / hd))
        return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s])
    # the oracle's (rounded) rotation agrees with the exact one within bf16 error
    for p in (0, 5, 63):
        np.testing.assert_allclose(om.apply_rope(q, cos[p], sin[p]), rot(q, p), atol=2e-2 * np.abs(q).max())
    assert abs(rot(q, 10) @ rot(k, 3) - rot(q, 27) @ rot(k, 20)) < 1e-9


def test_attention_matches_sdpa_gqa():
    rng = np.random.default_rng(2)
    H, Hkv, T, hd = 8, 2, 37, 16
    q = bf16_round(rng.standard_normal((H, hd)))
    K = bf16_round(rng.standard_normal((Hkv, T, hd)))
    V = bf16_round(rng.standard_normal((Hkv, T, hd)))
    got = om.attend(q, K, V, Hkv)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None, :, None, :],
                                         torch.from_numpy(K)[None], torch.from_numpy(V)[None],
                                         enable_gqa=True)[0, :, 0, :].numpy().reshape(-1)
    np.testing.assert_allclose(got, bf16_round(ref), rtol=0, atol=0)


@pytest.mark.parametrize("V", [1, 2, 7, 1024])
def test_softmax_top1_brute_force(V):
    rng = np.random.default_rng(V)
    x = rng.standard_normal(V) * 4
    got = om.softmax_top1(x[None])[0]
    ex = [math.exp(v) for v in x]
    want = max(ex) / math.fsum(ex)
    assert abs(got - want) <= 1e-14
    if V == 1:
        assert got == 1.0


def test_exit_head_matches_torch():
    from synth import ModelShape, make_weights
    sh = ModelShape(2, 64, 2, 2, 32, 64, 50, 32)
    w = make_weights(sh, 7)
    m = om.OracleModel(sh, w)
    h = np.random.default_rng(3).standard_normal((3, 64))
    p, logits = om.exit_head(m, 1, h)
    T = torch.from_numpy(m.w(1, "head_T"))
    E = torch.from_numpy(m.lm_head)
    hb = torch.from_numpy(bf16_round(h))
    z = torch.from_numpy(bf16_round((hb @ T.T).numpy()))
    ref = torch.softmax(z @ E.T, dim=-1).max(dim=-1).values.numpy()
    np.testing.assert_allclose(p, ref, rtol=1e-13)
