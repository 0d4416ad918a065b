"""CPU checks of the parity protocol's exit-head bound (tests/parity.py,
head_lnp_bound): a float32 evaluation of the head (float32 products and sums,
bf16 roundings of its input and of z, as the GPU computes it) from a hidden
state with a measured error stays within the bound derived from that error,
and the bound is far tighter than the worst case 4e-2 * max|logit|."""
import numpy as np
import pytest

import synth
from oracle import model as om
from oracle.numerics import bf16_round

import parity


def _head_f32(orc, layer, h):
    T = orc.w(layer, "head_T").astype(np.float32)
    E = orc.lm_head.astype(np.float32)
    a = bf16_round(h).astype(np.float32)
    z = bf16_round((T @ a).astype(np.float64)).astype(np.float32)
    lg = (E @ z).astype(np.float32)
    m = lg.max()
    return 1.0 / float(np.exp((lg - m).astype(np.float32)).astype(np.float32).sum(dtype=np.float32)), lg


@pytest.mark.parametrize("d,rel", [(256, 0.0), (256, 1e-4), (256, 3e-3), (4096, 0.0), (4096, 1e-3)])
def test_float32_head_within_derived_bound(d, rel):
    sh = synth.ModelShape(2, d, 4, 4, 64, 256, 3000, 32)
    w = synth.make_weights(sh, 9, alpha=np.array([40.0 if d == 256 else 4.0]))
    orc = om.OracleModel(sh, w)
    rng = np.random.default_rng(1)
    worst = 0.0
    for _ in range(4):
        h_o = rng.standard_normal(sh.d_model)
        h_g = h_o + rel * np.abs(h_o).max() * rng.standard_normal(sh.d_model)
        po, lo = om.exit_head(orc, 1, h_o[None])
        pg, _ = _head_f32(orc, 1, h_g)
        bound = parity.head_lnp_bound(orc, 1, h_g, h_o)
        assert abs(np.log(pg) - np.log(po[0])) <= bound
        worst = max(worst, bound / (4e-2 * np.abs(lo).max()))
    if rel <= 1e-4:   # the bound follows the measured error: far below the worst case when it is small
        assert worst < 0.2, worst
