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


# ---------------------------------------------------------------------------
# The exit head pinned by closed forms (AdaDecode explainer, section 2.1: the
# head's logits are h^(l) T^(l) E^T with E the LM-head matrix and no norm in
# between; section 2.2: its top-1 probability is what gamma is compared with).
# Each case builds weights for which the logits are known exactly, with
# - tok_emb (E_in) unlike lm_head (E): a head that used E_in fails;
# - h far from unit RMS and a final-norm gain of 3: a head that applied the
#   final RMSNorm (or its gain) fails;
# - values placed off the bf16 grid where a rounding matters: a head that
#   dropped either rounding (of h, or of z = T h) fails.
# ---------------------------------------------------------------------------
def _head_model(d, V, T, E, gain=3.0):
    from synth import ModelShape
    sh = ModelShape(2, d, 1, 1, 32, 32, V, 32)

    def bits(a):
        return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    rng = np.random.default_rng(11)
    w = {"tok_emb": bits(rng.standard_normal((V, d))), "lm_head": bits(E),
         "final_norm": bits(np.full(d, gain)), "layers": [{"head_T": bits(T)}, {}]}
    return om.OracleModel(sh, w)


def _p_closed(logits):
    """max softmax by fsum over exp(l - max): the textbook definition."""
    m = max(logits)
    return 1.0 / math.fsum(math.exp(v - m) for v in logits)


def _diag_E(d, V, c):
    E = np.zeros((V, d))
    E[np.arange(d), np.arange(d)] = c
    return E


def test_exit_head_identity_head_closed_form():
    """T = I, E = c [I; 0], h on the bf16 grid: logits are c h_v for v < d and 0 beyond."""
    d, V, c = 32, 80, 2.0
    h = (np.arange(d) - 11.0) * 0.25          # on the bf16 grid, RMS ~ 2.9
    m = _head_model(d, V, np.eye(d), _diag_E(d, V, c))
    p, logits = om.exit_head(m, 1, h[None])
    want = np.concatenate([c * h, np.zeros(V - d)])
    np.testing.assert_array_equal(logits[0], want)
    assert abs(p[0] - _p_closed(want.tolist())) <= 1e-15


def test_exit_head_orientation_of_T():
    """T a permutation (T[j, pi(j)] = 1): z_j = h_pi(j), so logit v is c h_pi(v) (z_j = sum_i T[j, i] h_i)."""
    d, V, c = 32, 48, 1.0
    pi = np.random.default_rng(4).permutation(d)
    T = np.zeros((d, d))
    T[np.arange(d), pi] = 1.0
    h = np.arange(d, dtype=np.float64) * 0.5
    m = _head_model(d, V, T, _diag_E(d, V, c))
    _, logits = om.exit_head(m, 1, h[None])
    np.testing.assert_array_equal(logits[0, :d], c * h[pi])
    # the transposed map would put h_v at pi(v): differs for a non-involution
    assert not np.array_equal(logits[0, :d], c * h[np.argsort(pi)])


def test_exit_head_rounds_its_input_to_bf16():
    """z_j = bf16(h_j) + h_{j+32} for j < 32 with h_j = m_j 2^-7 + 2^-9 (m_j in
    [128, 255]) and h_{j+32} = 2^-8: rounding h first gives bf16(h_j) = m_j 2^-7
    (a quarter unit rounds down), and the sum m_j 2^-7 + 2^-8 is the midpoint
    between two bf16 values, which rounds to the even one (torch's cast of the
    exact value).  Without the first rounding the sum lies above the midpoint
    and always rounds up, so the logits of even m_j differ."""
    d, V, c = 64, 100, 8.0
    mv = 128 + (np.arange(32) * 37) % 128
    h = np.concatenate([mv * 2.0 ** -7 + 2.0 ** -9, np.full(32, 2.0 ** -8)])
    T = np.eye(d)
    T[np.arange(32), np.arange(32) + 32] = 1.0
    m = _head_model(d, V, T, _diag_E(d, V, c))
    p, logits = om.exit_head(m, 1, h[None])
    zs = torch.from_numpy((mv * 2.0 ** -7 + 2.0 ** -8).astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(zs[mv % 2 == 0], mv[mv % 2 == 0] * 2.0 ** -7)   # ties went to even
    z = np.concatenate([zs, np.full(32, 2.0 ** -8)])
    want = np.concatenate([c * z, np.zeros(V - d)])
    np.testing.assert_array_equal(logits[0], want)
    assert abs(p[0] - _p_closed(want.tolist())) <= 1e-15


def test_exit_head_rounds_z_to_bf16():
    """T = 1.5 I and h_v = m_v 2^-7 with odd m_v in [129, 255]: 1.5 m_v needs 9
    significant bits, so z_v = bf16(1.5 h_v) (nearest, ties to even, from
    torch's float32 -> bfloat16 cast of the exact value) differs from 1.5 h_v."""
    d, V, c = 64, 90, 2.0
    mv = 129 + 2 * (np.arange(d) % 64)
    h = mv * 2.0 ** -7
    m = _head_model(d, V, 1.5 * np.eye(d), _diag_E(d, V, c))
    p, logits = om.exit_head(m, 1, h[None])
    z = torch.from_numpy((1.5 * h).astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.all(z != 1.5 * h)
    want = np.concatenate([c * z, np.zeros(V - d)])
    np.testing.assert_array_equal(logits[0], want)
    assert abs(p[0] - _p_closed(want.tolist())) <= 1e-15


def test_exit_head_zero_T_gives_uniform():
    """T = 0: every logit is 0 and p = 1 / V exactly."""
    d, V = 32, 1000
    rng = np.random.default_rng(5)
    m = _head_model(d, V, np.zeros((d, d)), rng.standard_normal((V, d)))
    p, logits = om.exit_head(m, 1, rng.standard_normal((3, d)))
    assert np.all(logits == 0)
    np.testing.assert_array_equal(p, np.full(3, 1.0 / V))


def test_exit_head_ignores_final_norm_gain():
    """The head has no final RMSNorm: changing the final-norm gain leaves p and the logits unchanged."""
    d, V = 32, 200
    rng = np.random.default_rng(6)
    T = rng.standard_normal((d, d)) * 0.2
    E = rng.standard_normal((V, d))
    h = rng.standard_normal((2, d)) * 7
    p1, l1 = om.exit_head(_head_model(d, V, T, E, gain=1.0), 1, h)
    p2, l2 = om.exit_head(_head_model(d, V, T, E, gain=0.25), 1, h)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(p1, p2)
