"""Pins of the oracle's bf16 rounding and int4 quantiser (CPU)."""
import numpy as np
import pytest
import torch

from oracle.numerics import bf16_round, from_bf16_bits
from oracle.quant import quantize_int4, dequantize_int4


def test_bf16_round_matches_torch_cast_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_round_ties_to_even_and_single_rounding():
    one = 1.0
    ulp = 2.0 ** -7
    # exact midpoints round to the even neighbour
    assert bf16_round(one + ulp / 2) == one
    assert bf16_round(one + 3 * ulp / 2) == one + 2 * ulp
    assert bf16_round(-(one + ulp / 2)) == -one
    # just above a midpoint (below float32 resolution of the midpoint) rounds up:
    # a detour through float32 would land on the midpoint and round down
    assert bf16_round(one + ulp / 2 + 2.0 ** -40) == one + ulp
    assert bf16_round(0.0) == 0.0
    assert np.isinf(bf16_round(3.5e38))


def test_from_bf16_bits():
    assert from_bf16_bits(np.array([0x3F80], np.uint16))[0] == 1.0
    assert from_bf16_bits(np.array([0xC000], np.uint16))[0] == -2.0
    assert from_bf16_bits(np.array([0x3C23], np.uint16))[0] == float(np.float32(
        np.array([0x3C230000], np.uint32).view(np.float32)[0]))


def _bf16_matrix(rng, n, k, std=0.02):
    return bf16_round(rng.standard_normal((n, k)) * std)


@pytest.mark.parametrize("group", [32, 128])
def test_int4_closed_form(group):
    rng = np.random.default_rng(1)
    w = _bf16_matrix(rng, 64, 4 * group)
    w[3, :group] = 0.0                      # a zero group
    q, s = quantize_int4(w, group)
    assert q.dtype == np.int8 and s.shape == (64, 4)
    # codes stay in [-7, 7] (the scale rounding can shift max|w|/s by < 2^-8 around 7)
    assert q.min() >= -7 and q.max() <= 7
    # scales are bf16 values and equal bf16(max|w| / 7)
    np.testing.assert_array_equal(bf16_round(s), s)
    wg = w.reshape(64, 4, group)
    amax = np.abs(wg).max(axis=2)
    np.testing.assert_array_equal(s, bf16_round(amax / 7))
    # the group maximum maps to +-7
    idx = np.abs(wg).argmax(axis=2)
    qg = q.reshape(64, 4, group)
    top = np.take_along_axis(qg, idx[:, :, None], 2)[:, :, 0]
    sign = np.sign(np.take_along_axis(wg, idx[:, :, None], 2)[:, :, 0])
    nz = amax > 0
    np.testing.assert_array_equal(top[nz], (7 * sign[nz]).astype(np.int8))
    # zero group
    assert s[3, 0] == 0 and np.all(q[3, :group] == 0)
    # dequantisation is q*s exactly and within half a step of w
    wh = dequantize_int4(q, s, group)
    np.testing.assert_array_equal(wh, (qg.astype(np.float64) * s[:, :, None]).reshape(64, -1))
    np.testing.assert_array_equal(wh.astype(np.float32).astype(np.float64), wh)  # exact in fp32
    err = np.abs(w - wh).reshape(64, 4, group)
    assert np.all(err <= s[:, :, None] / 2)


def test_int4_brute_force_nearest_code():
    """Every code is the nearest of the 16 codes to w/s, ties to the even code."""
    rng = np.random.default_rng(2)
    group = 32
    w = _bf16_matrix(rng, 16, 8 * group)
    # plant exact ties: w = (k + 1/2) * s for a group whose scale is known
    w[0, :group] = 0.0
    w[0, 0] = 7.0                      # scale bf16(1.0) = 1.0
    w[0, 1] = 2.5
    w[0, 2] = -3.5
    w[0, 3] = 0.5
    q, s = quantize_int4(w, group)
    assert s[0, 0] == 1.0
    assert (q[0, 1], q[0, 2], q[0, 3]) == (2, -4, 0)
    codes = np.arange(-8, 8, dtype=np.float64)
    for n in range(w.shape[0]):
        for k in range(w.shape[1]):
            sc = s[n, k // group]
            if sc == 0:
                assert q[n, k] == 0
                continue
            d = np.abs(w[n, k] - codes * sc)
            best = codes[d == d.min()]
            want = best[0] if len(best) == 1 else best[np.argmin(np.abs(best) % 2)]
            assert q[n, k] == want, (n, k)


def test_int4_size_matches_page_reduction():
    """W4A16 copies are about 75% smaller than 16-bit weights (River-LLM section 4.2):
    int4 codes plus one bf16 scale per 128 weights take 0.2578 of the bf16 bytes."""
    K, G = 4096, 128
    frac = (K / 2 + 2 * K / G) / (2 * K)
    assert abs((1 - frac) - 0.75) < 0.01
