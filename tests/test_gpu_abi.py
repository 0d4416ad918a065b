"""GPU tests of the C ABI: int4 copies bit-exact vs the oracle, error paths, self-consistency."""
import numpy as np
import pytest

import synth
from synth import ModelShape
from oracle.quant import quantize_int4
from oracle.numerics import from_bf16_bits

pytestmark = pytest.mark.gpu

ODD = ModelShape(3, 160, 5, 1, 32, 224, 1003, 32, rope_theta=500000.0)
MID = ModelShape(3, 2048, 16, 4, 128, 5120, 5000, 128, rope_theta=500000.0)
G64 = ModelShape(2, 4352, 32, 2, 128, 2176, 300, 64)   # K = 4352: two full int4 blocks + a 256 tail


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_shared_exit_amd import api as A
    return A


def _model(api, sh, seed=3, alpha=None, **kw):
    w = synth.make_weights(sh, seed, alpha=alpha)
    dev = api.upload_weights(w)
    return w, api.Model(sh, dev, **kw)


@pytest.mark.parametrize("sh", [ODD, MID, G64], ids=["odd", "mid", "g64"])
def test_int4_copies_bit_exact(api, sh):
    w, m = _model(api, sh, max_batch=2, max_positions=8)
    try:
        for l in range(2, sh.n_layers + 1):
            for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
                codes, scales = m.exit_weights(l, name)
                q, s = quantize_int4(from_bf16_bits(w["layers"][l - 1][name]), sh.group)
                np.testing.assert_array_equal(codes, q, err_msg=f"codes layer {l} {name}")
                np.testing.assert_array_equal(from_bf16_bits(scales), s, err_msg=f"scales layer {l} {name}")
    finally:
        m.close()


def test_error_paths_leave_state_unchanged(api):
    from kv_shared_exit_amd import _binding as B
    sh = ODD
    w, m = _model(api, sh, max_batch=2, max_positions=8)
    c = api.KVCache(m, 2, 6, track=True)
    try:
        prompts = np.array([[1, 2, 3], [4, 5, 6]], np.int32)
        api.prefill(m, c, prompts)
        assert list(c.lengths()) == [3, 3]
        with pytest.raises(B.EEError) as e:
            api.decode_step(m, c, 2, tokens=[1, sh.vocab])
        assert e.value.status == B.EE_ERR_INVALID_ARG
        with pytest.raises(B.EEError) as e:
            api.decode_step(m, c, 2, tokens=[1, 2], forced=[0, sh.n_layers + 1])
        assert e.value.status == B.EE_ERR_INVALID_ARG
        with pytest.raises(B.EEError) as e:
            api.decode_step(m, c, 3, tokens=[1, 2, 3])
        assert e.value.status == B.EE_ERR_INVALID_ARG
        with pytest.raises(B.EEError) as e:
            api.prefill(m, c, np.zeros((2, 4), np.int32))   # 3 + 4 > 6
        assert e.value.status == B.EE_ERR_CACHE_FULL
        assert list(c.lengths()) == [3, 3]
        for _ in range(3):
            api.decode_step(m, c, 2)
        assert list(c.lengths()) == [6, 6]
        with pytest.raises(B.EEError) as e:
            api.decode_step(m, c, 2)
        assert e.value.status == B.EE_ERR_CACHE_FULL
        assert list(c.lengths()) == [6, 6]
        occ = c.occupancy()
        assert np.all(occ[:, :, :6] == 1)
        c.reset(1)
        assert list(c.lengths()) == [6, 0]
        with pytest.raises(B.EEError) as e:
            c.read(1, 1, 0, 1)
        assert e.value.status == B.EE_ERR_NOT_WRITTEN
        k, v = c.read(2, 0, 0, 6)
        assert k.shape == (6, sh.n_kv_heads, sh.head_dim)
        # a model with live caches cannot be destroyed
        with pytest.raises(B.EEError):
            m.close()
    finally:
        c.close()
        m.close()


def test_kept_tokens_are_per_cache_and_dropped_by_rollback(api):
    """A step without input tokens feeds each sequence the last output token of
    the same cache: two caches on one model keep their own, equal to passing
    those tokens explicitly on fresh caches.  After a rollback or a reset the
    kept token no longer follows the sequence's last position, so a step
    without tokens is refused (state unchanged) until tokens are passed again."""
    from kv_shared_exit_amd import _binding as B
    sh = ODD
    w, m = _model(api, sh, alpha=np.full(sh.n_layers - 1, 3000.0), max_batch=2, max_positions=12)
    pa = np.array([[5, 6, 7], [8, 9, 10]], np.int32)
    pb = np.array([[100, 200, 300], [400, 500, 600]], np.int32)
    ca, cb = api.KVCache(m, 2, 12), api.KVCache(m, 2, 12)
    fresh = api.KVCache(m, 2, 12)
    try:
        with pytest.raises(B.EEError) as e:
            api.decode_step(m, fresh, 2)          # nothing produced on this cache yet
        assert e.value.status == B.EE_ERR_INVALID_ARG
        ta0, tb0 = api.prefill(m, ca, pa), api.prefill(m, cb, pb)
        ta1, ea1 = api.decode_step(m, ca, 2)
        tb1, eb1 = api.decode_step(m, cb, 2)
        ta2, ea2 = api.decode_step(m, ca, 2)
        # the same steps with explicit tokens on fresh caches
        ra, rb = api.KVCache(m, 2, 12), api.KVCache(m, 2, 12)
        try:
            api.prefill(m, ra, pa)
            api.prefill(m, rb, pb)
            t, e_ = api.decode_step(m, ra, 2, tokens=ta0)
            np.testing.assert_array_equal(t, ta1)
            np.testing.assert_array_equal(e_, ea1)
            t, e_ = api.decode_step(m, rb, 2, tokens=tb0)
            np.testing.assert_array_equal(t, tb1)
            np.testing.assert_array_equal(e_, eb1)
            t, e_ = api.decode_step(m, ra, 2, tokens=ta1)
            np.testing.assert_array_equal(t, ta2)
            np.testing.assert_array_equal(e_, ea2)
        finally:
            ra.close()
            rb.close()
        ca.rollback(-1, 1)
        assert list(ca.lengths()) == [4, 4]
        with pytest.raises(B.EEError) as e:
            api.decode_step(m, ca, 2)
        assert e.value.status == B.EE_ERR_INVALID_ARG
        assert list(ca.lengths()) == [4, 4]
        t, _ = api.decode_step(m, ca, 2, tokens=ta1)  # the rolled-back step again
        np.testing.assert_array_equal(t, ta2)
        api.decode_step(m, ca, 2)                     # kept again
        assert list(ca.lengths()) == [6, 6]
        cb.reset(0)
        with pytest.raises(B.EEError) as e:
            api.decode_step(m, cb, 2)
        assert e.value.status == B.EE_ERR_INVALID_ARG
    finally:
        fresh.close()
        ca.close()
        cb.close()
        m.close()


def test_cache_without_tracking_has_no_occupancy(api):
    from kv_shared_exit_amd import _binding as B
    w, m = _model(api, ODD, max_batch=1, max_positions=4)
    c = api.KVCache(m, 1, 4, track=False, torch_buffer=False)
    try:
        with pytest.raises(B.EEError) as e:
            c.occupancy()
        assert e.value.status == B.EE_ERR_UNSUPPORTED
    finally:
        c.close()
        m.close()


def _run(api, sh, w, mode, gamma, B_, P, steps, forced=None, graph=False, kv=None):
    import torch
    dev = api.upload_weights(w)
    m = api.Model(sh, dev, gamma=gamma, exit_mode=mode, max_batch=B_, max_positions=P + steps + 1)
    c = api.KVCache(m, B_, P + steps + 1)
    prompts = np.random.default_rng(7).integers(0, sh.vocab, (B_, P)).astype(np.int32)
    st = torch.cuda.Stream()
    out = []
    try:
        tok = api.prefill(m, c, prompts, stream=st)
        for s in range(steps):
            dbg = {"logits": None, "p": None} if not graph else None
            t, e = api.decode_step(m, c, B_, forced=None if forced is None else forced(s),
                                   stream=st, debug=dbg)
            out.append((t.copy(), e.copy(), None if dbg is None else dbg["logits"].copy()))
        if kv is not None:
            for l in range(1, sh.n_layers + 1):
                for b in range(B_):
                    kv.append(c.read(l, b, 0, P + steps))
    finally:
        c.close()
        m.close()
    return out


def test_no_exit_equals_unquantised_exit_copies_bitwise(api):
    """gamma > 1 (nobody exits) and unquantised exit copies run the same arithmetic: bitwise equal."""
    from kv_shared_exit_amd import _binding as B
    sh = MID
    w = synth.make_weights(sh, 5, alpha=np.full(sh.n_layers - 1, 1e3))
    a = _run(api, sh, w, B.EE_EXIT_INT4, 1.5, 3, 6, 4)
    b = _run(api, sh, w, B.EE_EXIT_BF16, 0.1, 3, 6, 4)
    for (ta, ea, la), (tb, eb, lb) in zip(a, b):
        assert np.all(ea == sh.n_layers)
        np.testing.assert_array_equal(ta, tb)
        np.testing.assert_array_equal(la, lb)


def test_plain_decoder_mode_equals_no_exit_bitwise(api):
    """EE_EXIT_NONE (the baseline: no exit heads, full depth) runs the same layer
    arithmetic as the exit-head model when nobody exits (gamma > 1): tokens and
    final logits bitwise equal, every exit layer = L; it needs no head weights,
    and the graph-replayed step gives the same tokens."""
    from kv_shared_exit_amd import _binding as B
    sh = MID
    w = synth.make_weights(sh, 5, alpha=np.full(sh.n_layers - 1, 1e3))
    a = _run(api, sh, w, B.EE_EXIT_INT4, 1.5, 3, 6, 4)
    w_nohead = {k: v for k, v in w.items() if k != "layers"}
    w_nohead["layers"] = [{k: v for k, v in lw.items() if k != "head_T"} for lw in w["layers"]]
    b = _run(api, sh, w_nohead, B.EE_EXIT_NONE, None, 3, 6, 4)
    g = _run(api, sh, w_nohead, B.EE_EXIT_NONE, None, 3, 6, 4, graph=True)
    for (ta, ea, la), (tb, eb, lb), (tg, eg, _) in zip(a, b, g):
        assert np.all(ea == sh.n_layers) and np.all(eb == sh.n_layers) and np.all(eg == sh.n_layers)
        np.testing.assert_array_equal(ta, tb)
        np.testing.assert_array_equal(la, lb)
        np.testing.assert_array_equal(tb, tg)


def test_plain_decoder_mode_has_no_exit_copies(api):
    from kv_shared_exit_amd import _binding as B
    w, m = _model(api, ODD, exit_mode=B.EE_EXIT_NONE, max_batch=1, max_positions=4)
    try:
        with pytest.raises(B.EEError) as e:
            m.exit_weights(2, "wq")
        assert e.value.status == B.EE_ERR_UNSUPPORTED
    finally:
        m.close()


def test_two_runs_are_bitwise_identical(api):
    from kv_shared_exit_amd import _binding as B
    sh = ODD
    w = synth.make_weights(sh, 6, alpha=np.full(sh.n_layers - 1, 3000.0))
    rng = lambda s: np.random.default_rng(s).integers(0, sh.n_layers + 1, 4).astype(np.int32)
    a = _run(api, sh, w, B.EE_EXIT_INT4, 0.75, 4, 5, 6, forced=rng)
    b = _run(api, sh, w, B.EE_EXIT_INT4, 0.75, 4, 5, 6, forced=rng)
    for (ta, ea, la), (tb, eb, lb) in zip(a, b):
        np.testing.assert_array_equal(ta, tb)
        np.testing.assert_array_equal(ea, eb)
        np.testing.assert_array_equal(la, lb)


def test_rollback_then_replay_is_identical(api):
    from kv_shared_exit_amd import _binding as B
    sh = ODD
    w, m = _model(api, sh, alpha=np.full(sh.n_layers - 1, 3000.0), max_batch=3, max_positions=16)
    c = api.KVCache(m, 3, 16, track=True)
    try:
        api.prefill(m, c, np.array([[5, 6, 7], [8, 9, 10], [11, 12, 13]], np.int32))
        toks = np.array([1, 2, 3], np.int32)
        d1 = {"logits": None}
        t1, e1 = api.decode_step(m, c, 3, tokens=toks, debug=d1)
        k1, v1 = c.read(2, 1, 0, 4)
        c.rollback(-1, 1)
        assert list(c.lengths()) == [3, 3, 3]
        assert np.all(c.occupancy()[:, :, 3] == 0)
        d2 = {"logits": None}
        t2, e2 = api.decode_step(m, c, 3, tokens=toks, debug=d2)
        np.testing.assert_array_equal(t1, t2)
        np.testing.assert_array_equal(e1, e2)
        np.testing.assert_array_equal(d1["logits"], d2["logits"])
        k2, v2 = c.read(2, 1, 0, 4)
        np.testing.assert_array_equal(k1, k2)
        assert np.all(c.occupancy()[:, :, :4] == 1)
        with pytest.raises(B.EEError) as e:
            c.rollback(0, 5)
        assert e.value.status == B.EE_ERR_INVALID_ARG
    finally:
        c.close()
        m.close()


def test_graph_replay_equals_eager(api):
    """Steps without debug outputs replay a captured graph; with them the kernels
    are launched one by one.  Both must give the same tokens, exits and K/V."""
    from kv_shared_exit_amd import _binding as B
    sh = MID
    w = synth.make_weights(sh, 8, alpha=np.full(sh.n_layers - 1, 3000.0))
    forced = lambda s: np.random.default_rng(100 + s).integers(0, sh.n_layers + 1, 5).astype(np.int32)
    kva, kvb = [], []
    a = _run(api, sh, w, B.EE_EXIT_INT4, 0.75, 5, 6, 5, forced=forced, graph=False, kv=kva)
    b = _run(api, sh, w, B.EE_EXIT_INT4, 0.75, 5, 6, 5, forced=forced, graph=True, kv=kvb)
    for (ta, ea, _), (tb, eb, _) in zip(a, b):
        np.testing.assert_array_equal(ta, tb)
        np.testing.assert_array_equal(ea, eb)
    for (ka, va), (kb, vb) in zip(kva, kvb):
        np.testing.assert_array_equal(ka, kb)
        np.testing.assert_array_equal(va, vb)


def test_sampled_decoding_configuration_errors(api):
    """Sampled decoding drafts from the exit head after every layer; other
    configurations are refused at creation (any batch size is accepted)."""
    from kv_shared_exit_amd import _binding as B
    w = synth.make_weights(ODD, 3)
    dev = api.upload_weights(w)
    cases = [(dict(temperature=1.0, criterion=B.EE_CRIT_STS), B.EE_ERR_INVALID_ARG),
             (dict(temperature=1.0, check_every=2), B.EE_ERR_INVALID_ARG),
             (dict(temperature=1.0, exit_mode=B.EE_EXIT_NONE), B.EE_ERR_INVALID_ARG),
             (dict(temperature=-1.0), B.EE_ERR_INVALID_ARG),
             (dict(temperature=float("nan")), B.EE_ERR_INVALID_ARG)]
    for kw, status in cases:
        with pytest.raises(B.EEError) as e:
            api.Model(ODD, dev, max_positions=8, **{"max_batch": 2, **kw})
        assert e.value.status == status, kw


def test_sampled_graph_replay_equals_eager_and_repeats(api):
    """Sampled steps replay their captured graph (the resampling pass included)
    with the same tokens as eager launches, and a rolled-back step draws the
    same tokens again (the draws are keyed by sequence and position)."""
    sh = ODD
    w, m = _model(api, sh, alpha=np.full(sh.n_layers - 1, 40.0), max_batch=4, max_positions=16,
                  gamma=0.3, temperature=1.0, sample_seed=7)
    c = api.KVCache(m, 4, 16)
    try:
        api.prefill(m, c, np.arange(20, dtype=np.int32).reshape(4, 5))
        toks = np.array([1, 2, 3, 4], np.int32)
        runs = []
        for debug in (None, {"gap": None}, None):
            t, e = api.decode_step(m, c, 4, tokens=toks, debug=debug)
            runs.append((t.copy(), e.copy()))
            c.rollback(-1, 1)
        for t, e in runs[1:]:
            np.testing.assert_array_equal(t, runs[0][0])
            np.testing.assert_array_equal(e, runs[0][1])
    finally:
        c.close()
        m.close()
