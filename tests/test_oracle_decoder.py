"""Whole-step pins of the oracle: special cases that reduce to a plain decoder, and invariants."""
import numpy as np
import pytest
import torch

import synth
from synth import ModelShape
from oracle import model as om
from oracle.quant import quantize_int4, dequantize_int4
from oracle.numerics import from_bf16_bits
from plain_decoder import PlainDecoder, bf16_tensor

NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")

SHAPES = {
    "tiny": synth.TINY,
    # grouped heads, head_dim 16, widths that are not powers of two
    "gqa_odd": ModelShape(3, 96, 6, 2, 16, 160, 300, 32, rope_theta=500000.0),
}


def _setup(name, seed=11, exit_mode="int4", alpha=None):
    sh = SHAPES[name]
    w = synth.make_weights(sh, seed, alpha=alpha)
    return sh, w, om.OracleModel(sh, w, exit_mode=exit_mode)


def _plain(sh, w, dequant_layers=()):
    layers = []
    for l in range(1, sh.n_layers + 1):
        lw = {n: bf16_tensor(w["layers"][l - 1][n]) for n in NAMES}
        if l in dequant_layers:
            for n in om.LINEAR:
                q, s = quantize_int4(from_bf16_bits(w["layers"][l - 1][n]), sh.group)
                lw[n] = torch.from_numpy(dequantize_int4(q, s, sh.group))
        layers.append(lw)
    return PlainDecoder(sh, bf16_tensor(w["tok_emb"]), bf16_tensor(w["lm_head"]),
                        bf16_tensor(w["final_norm"]), layers)


def _prompt(sh, n, seed=0):
    return np.random.default_rng(seed).integers(0, sh.vocab, n)


@pytest.mark.parametrize("name", list(SHAPES))
def test_gamma_above_one_is_the_plain_decoder(name):
    sh, w, m = _setup(name)
    P, steps = 9, 6
    prompt = _prompt(sh, P)
    cache = om.KVCache(sh, 1, P + steps + 1)
    toks, exits = om.generate(m, cache, prompt[None], steps, gamma=1.5)
    assert np.all(exits == sh.n_layers)
    ref, gaps = _plain(sh, w).greedy(prompt, steps)
    for t in range(steps + 1):
        if gaps[t] > 1e-9:
            assert toks[0, t] == ref[t], t
        else:
            break
    # hidden states and KV of the whole sequence agree with the full causal pass
    seq = list(prompt) + list(toks[0, :-1])
    hid, logits, K, V = _plain(sh, w).forward(seq)
    n = len(seq)
    np.testing.assert_allclose(cache.K[:, 0, :, :n], K.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(cache.V[:, 0, :, :n], V.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", list(SHAPES))
def test_gamma_nonpositive_exits_after_layer_one(name):
    """gamma <= 0 exits after layer 1 at every step.  Decoding from an empty cache, every
    position then runs layers 2..L as dequantised copies, so the whole sequence equals a plain
    decoder whose layers 2..L are the dequantised weights."""
    sh, w, m = _setup(name)
    steps = 7
    first = int(_prompt(sh, 1, 1)[0])
    cache = om.KVCache(sh, 1, steps + 2)
    toks = [first]
    for s in range(steps):
        t, e, _ = om.decode_step(m, cache, [toks[-1]], gamma=0.0)
        assert e[0] == 1
        toks.append(int(t[0]))
    quant = _plain(sh, w, dequant_layers=range(2, sh.n_layers + 1))
    ref, gaps = quant.greedy([first], steps - 1)
    for t in range(steps):
        if gaps[t] <= 1e-9:
            break
        assert toks[t + 1] == ref[t], t
    _, _, K, V = quant.forward(toks[:-1])
    np.testing.assert_allclose(cache.K[:, 0, :, :steps], K.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(cache.V[:, 0, :, :steps], V.numpy(), rtol=0, atol=1e-12)


def test_forced_exit_uses_dequantised_layers_and_shared_slots():
    """After a forced exit at layer e the KV of layers e+1..L are the dequantised layers' K/V."""
    sh, w, m = _setup("gqa_odd")
    L = sh.n_layers
    # single token, no history: the step equals a length-1 causal pass
    for e in range(1, L + 1):
        cache = om.KVCache(sh, 1, 4)
        tok = _prompt(sh, 1, 5)
        t, ex, info = om.decode_step(m, cache, tok, forced=[e], trace=True)
        assert ex[0] == e
        ref = _plain(sh, w, dequant_layers=range(e + 1, L + 1))
        hid, logits, K, V = ref.forward(list(tok))
        np.testing.assert_allclose(info["hidden"][0], hid.numpy()[:, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(cache.K[:, 0, :, :1], K.numpy(), atol=1e-12)
        np.testing.assert_allclose(cache.V[:, 0, :, :1], V.numpy(), atol=1e-12)
        assert t[0] == int(torch.argmax(logits[0]))
        # heads ran on layers 1..e (the sequence was on the backbone), not after
        assert np.all(np.isfinite(info["p"][0, :min(e, L - 1)]))
        assert np.all(np.isnan(info["p"][0, e:]))


@pytest.mark.parametrize("gamma", [0.0, 0.5, 0.9])
def test_unquantised_exit_copies_equal_full_depth(gamma):
    sh = SHAPES["gqa_odd"]
    w = synth.make_weights(sh, 3, alpha=np.full(sh.n_layers - 1, 3000.0))
    P, steps = 5, 6
    prompt = _prompt(sh, P, 2)
    a = om.OracleModel(sh, w, exit_mode="bf16")
    b = om.OracleModel(sh, w, exit_mode="bf16")
    ca, cb = om.KVCache(sh, 1, 16), om.KVCache(sh, 1, 16)
    ta, ea = om.generate(a, ca, prompt[None], steps, gamma=gamma)
    tb, eb = om.generate(b, cb, prompt[None], steps, gamma=2.0)
    np.testing.assert_array_equal(ta, tb)
    np.testing.assert_array_equal(ca.K, cb.K)
    assert np.all(eb == sh.n_layers)


def test_every_slot_written_once_and_batch_independence():
    sh = SHAPES["gqa_odd"]
    w = synth.make_weights(sh, 4, alpha=np.full(sh.n_layers - 1, 3000.0))
    m = om.OracleModel(sh, w)
    B, P, steps = 3, 4, 8
    prompts = np.stack([_prompt(sh, P, 10 + b) for b in range(B)])
    cache = om.KVCache(sh, B, 16)
    toks, exits = om.generate(m, cache, prompts, steps, gamma=0.6)
    n = P + steps
    assert np.all(cache.occ[:, :, :n] == 1) and np.all(cache.occ[:, :, n:] == 0)
    assert len(np.unique(exits)) > 1          # exits diverge inside the batch
    for b in range(B):
        c1 = om.KVCache(sh, 1, 16)
        t1, e1 = om.generate(m, c1, prompts[b:b + 1], steps, gamma=0.6)
        np.testing.assert_array_equal(t1[0], toks[b])
        np.testing.assert_array_equal(e1[0], exits[b])
        np.testing.assert_array_equal(c1.K[:, 0], cache.K[:, b])


def test_prefill_equals_token_by_token_full_depth():
    sh = SHAPES["gqa_odd"]
    w = synth.make_weights(sh, 5)
    m = om.OracleModel(sh, w)
    prompt = _prompt(sh, 6, 3)
    c1 = om.KVCache(sh, 1, 8)
    t1, info = om.prefill(m, c1, prompt[None], trace=True)
    c2 = om.KVCache(sh, 1, 8)
    for tok in prompt:
        t2, e2, i2 = om.decode_step(m, c2, [tok], gamma=2.0, trace=True)
    np.testing.assert_array_equal(c1.K, c2.K)
    np.testing.assert_array_equal(c1.V, c2.V)
    assert t1[0] == t2[0]
    np.testing.assert_allclose(info["hidden"][0, -1], i2["hidden"][0], rtol=0, atol=1e-12)


def test_first_step_exit_layer_monotone_in_gamma():
    sh = SHAPES["tiny"]
    w = synth.make_weights(sh, 6, alpha=np.full(sh.n_layers - 1, 3000.0))
    m = om.OracleModel(sh, w)
    prompt = _prompt(sh, 5, 4)
    last = 0
    for g in np.linspace(0.0, 1.0, 11):
        c = om.KVCache(sh, 1, 8)
        tok, _ = om.prefill(m, c, prompt[None])
        _, e, _ = om.decode_step(m, c, tok, gamma=g)
        assert e[0] >= last
        last = e[0]
    assert last == sh.n_layers
