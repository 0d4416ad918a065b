"""Pins of the oracle's prefill with River-LLM's sequence-level exit (River-LLM
explainer, section 6.1: in the prefill every token of a sequence leaves at the
same layer; section 5.2: when the smallest state transition similarity of the
tokens exceeds tau).  The reference is the plain decoder written from torch
library calls (tests/plain_decoder.py): its full causal pass gives the
similarities (torch normalisation) that decide the exit layer, and a plain
decoder whose layers after the exit are the dequantised int4 copies gives the
logits and K/V the prefill must reproduce."""
import numpy as np
import pytest
import torch

import synth
from synth import ModelShape
from oracle import model as om
from oracle.numerics import from_bf16_bits
from oracle.quant import quantize_int4, dequantize_int4
from plain_decoder import PlainDecoder, bf16_tensor

SH = ModelShape(4, 96, 6, 2, 16, 160, 300, 32, rope_theta=500000.0)
NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")
P = 7


def _plain(w, dequant_layers=()):
    layers = []
    for l in range(1, SH.n_layers + 1):
        lw = {n: bf16_tensor(w["layers"][l - 1][n]) for n in NAMES}
        if l in dequant_layers:
            for n in om.LINEAR:
                q, s = quantize_int4(from_bf16_bits(w["layers"][l - 1][n]), SH.group)
                lw[n] = torch.from_numpy(dequantize_int4(q, s, SH.group))
        layers.append(lw)
    return PlainDecoder(SH, bf16_tensor(w["tok_emb"]), bf16_tensor(w["lm_head"]),
                        bf16_tensor(w["final_norm"]), layers)


def _min_similarity(hidden):
    """[L] smallest cosine over the tokens between each layer's input and output (torch)."""
    out = []
    for l in range(1, hidden.shape[0]):
        a = torch.nn.functional.normalize(hidden[l - 1], dim=-1)
        b = torch.nn.functional.normalize(hidden[l], dim=-1)
        out.append(float((a * b).sum(-1).min()))
    return np.array(out)


def _prefill(w, prompts, tau):
    m = om.OracleModel(SH, w)
    c = om.KVCache(SH, len(prompts), P + 1)
    tok, info = om.prefill(m, c, prompts, exit_tau=tau)
    return tok, info, c


@pytest.fixture(scope="module")
def setup():
    w = synth.make_weights(SH, 17)
    prompts = np.random.default_rng(5).integers(0, SH.vocab, (2, P))
    return w, prompts


def _check_against_plain(w, prompt, e, info, cache, b):
    ref = _plain(w, dequant_layers=range(e + 1, SH.n_layers + 1))
    _, logits, K, V = ref.forward(list(prompt))
    np.testing.assert_allclose(info["logits"][b], logits[-1].numpy(), rtol=0, atol=1e-9)
    np.testing.assert_allclose(cache.K[:, b, :, :P], K.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(cache.V[:, b, :, :P], V.numpy(), rtol=0, atol=1e-12)


def test_unreachable_threshold_is_the_full_depth_prefill(setup):
    w, prompts = setup
    t1, i1, c1 = _prefill(w, prompts, 1.0)   # a cosine never exceeds 1
    t0, i0, c0 = _prefill(w, prompts, None)
    assert np.all(i1["exit"] == SH.n_layers)
    np.testing.assert_array_equal(t1, t0)
    np.testing.assert_array_equal(i1["logits"], i0["logits"])
    np.testing.assert_array_equal(c1.K, c0.K)
    for b in range(2):
        _check_against_plain(w, prompts[b], SH.n_layers, i1, c1, b)


def test_threshold_below_minus_one_exits_after_layer_one(setup):
    w, prompts = setup
    _, info, cache = _prefill(w, prompts, -1.5)
    np.testing.assert_array_equal(info["exit"], [1, 1])
    for b in range(2):
        _check_against_plain(w, prompts[b], 1, info, cache, b)


@pytest.mark.parametrize("layer", [1, 2, 3])
def test_exit_at_the_first_layer_whose_token_minimum_passes(setup, layer):
    """Thresholds just below sequence 0's token minimum at `layer` (unreachable
    elsewhere): sequence 0 leaves there; sequence 1 leaves there only if its own
    minimum also passes, else it runs full depth; each equals the plain decoder
    with dequantised layers after its exit."""
    w, prompts = setup
    mins = [_min_similarity(_plain(w).forward(list(prompts[b]))[0]) for b in range(2)]
    tau = np.full(SH.n_layers - 1, 2.0)
    tau[layer - 1] = mins[0][layer - 1] - 1e-9
    _, info, cache = _prefill(w, prompts, tau)
    want1 = layer if mins[1][layer - 1] > tau[layer - 1] else SH.n_layers
    np.testing.assert_array_equal(info["exit"], [layer, want1])
    for b, e in enumerate((layer, want1)):
        _check_against_plain(w, prompts[b], e, info, cache, b)
    # a threshold just above the minimum keeps sequence 0 on the backbone
    tau[layer - 1] = mins[0][layer - 1] + 1e-9
    _, info2, _ = _prefill(w, prompts[:1], tau)
    assert info2["exit"][0] == SH.n_layers


def test_sequences_are_independent(setup):
    w, prompts = setup
    mins = [_min_similarity(_plain(w).forward(list(prompts[b]))[0])[:SH.n_layers - 1] for b in range(2)]
    # between the two sequences' minima after layer 1 (one leaves there), below
    # both after layer 2 (the other leaves there)
    assert mins[0][0] != mins[1][0]
    tau = np.full(SH.n_layers - 1, 2.0)
    tau[0] = 0.5 * (mins[0][0] + mins[1][0])
    tau[1] = min(mins[0][1], mins[1][1]) - 1e-9
    _, both, cb = _prefill(w, prompts, tau)
    assert sorted(both["exit"].tolist()) == [1, 2]
    for b in range(2):
        _, one, c1 = _prefill(w, prompts[b:b + 1], tau)
        assert one["exit"][0] == both["exit"][b]
        np.testing.assert_array_equal(one["logits"][0], both["logits"][b])
        np.testing.assert_array_equal(c1.K[:, 0], cb.K[:, b])
