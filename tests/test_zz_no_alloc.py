"""The decode step for callers that cannot allocate (ee_decode_step_static)
against ee_decode_step: the same kernels over workspaces taken from the
library's static device array instead of the model's buffers, so tokens,
exit layers, K/V and occupancy must be bitwise equal.  Two calls in a row,
the second with a smaller batch (the array keeps the first call's contents),
then a third without input tokens; for the exit-head and similarity criteria,
sampled decoding, and a batch above 8 on the matrix-core passes.  A step
whose workspaces exceed the array is refused and changes nothing."""
import numpy as np
import pytest

import synth
from synth import ModelShape

pytestmark = pytest.mark.gpu

MID = ModelShape(3, 2048, 16, 4, 128, 5120, 5000, 128, rope_theta=500000.0)
ODD = ModelShape(3, 160, 5, 1, 32, 224, 1003, 32, rope_theta=500000.0)
WIDE = ModelShape(2, 256, 4, 2, 64, 512, 1000, 32)


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_shared_exit_amd import api as A
    return A


CASES = {
    "mid-head": dict(sh=MID, Bm=6, kw=dict(gamma=0.75), alpha=3000.0),
    "odd-sts": dict(sh=ODD, Bm=4, kw=dict(gamma=0.3, criterion=1), alpha=None),
    "odd-sampled": dict(sh=ODD, Bm=4, kw=dict(gamma=0.3, temperature=1.0, sample_seed=5), alpha=40.0),
    "wide-12": dict(sh=WIDE, Bm=12, kw=dict(gamma=0.75), alpha=3000.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_static_step_equals_decode_step(api, name):
    import torch
    case = CASES[name]
    sh, Bm = case["sh"], case["Bm"]
    L = sh.n_layers
    alpha = None if case["alpha"] is None else np.full(L - 1, case["alpha"])
    w = synth.make_weights(sh, 21, alpha=alpha)
    dev = api.upload_weights(w)
    P, S = 5, 12
    m = api.Model(sh, dev, max_batch=Bm, max_positions=S, **case["kw"])
    ref, sta = api.KVCache(m, Bm, S, track=True), api.KVCache(m, Bm, S, track=True)
    stream = torch.cuda.Stream()
    try:
        prompts = np.random.default_rng(3).integers(0, sh.vocab, (Bm, P)).astype(np.int32)
        t0 = api.prefill(m, ref, prompts, stream=stream)
        np.testing.assert_array_equal(api.prefill(m, sta, prompts, stream=stream), t0)
        rng = np.random.default_rng(4)
        forced = rng.integers(0, L + 1, Bm).astype(np.int32)
        forced[: Bm // 2] = 0          # half the rows decide by the criterion
        # call 1: the whole batch; call 2: a smaller batch; call 3: kept tokens
        calls = [(Bm, t0, forced), (Bm - 2, None, forced[: Bm - 2]), (Bm - 3, None, None)]
        prev = t0
        for i, (b, tok, frc) in enumerate(calls):
            if tok is None and i == 1:
                tok = prev[:b]
            tr, er = api.decode_step(m, ref, b, tokens=tok, forced=frc, stream=stream)
            ts, es = api.decode_step_static(m, sta, b, tokens=tok, forced=frc, stream=stream)
            np.testing.assert_array_equal(ts, tr, err_msg=f"{name} call {i + 1} tokens")
            np.testing.assert_array_equal(es, er, err_msg=f"{name} call {i + 1} exit layers")
            prev = tr
            print(f"[{name}] call {i + 1} batch {b}: tokens {tr.tolist()} exits {er.tolist()}", flush=True)
        np.testing.assert_array_equal(sta.lengths(), ref.lengths())
        np.testing.assert_array_equal(sta.occupancy(), ref.occupancy())
        n = P + 3
        for l in range(1, L + 1):
            for b in range(Bm):
                k1, v1 = ref.read(l, b, 0, int(ref.lengths()[b]))
                k2, v2 = sta.read(l, b, 0, int(sta.lengths()[b]))
                np.testing.assert_array_equal(k2, k1, err_msg=f"{name} K layer {l} seq {b}")
                np.testing.assert_array_equal(v2, v1, err_msg=f"{name} V layer {l} seq {b}")
        assert int(ref.lengths().max()) == n
    finally:
        ref.close()
        sta.close()
        m.close()


def test_static_step_refuses_workspaces_beyond_the_array(api):
    """With a feed-forward width of 49152 (d 4096) a batch of 16 runs the
    matrix-core passes, whose gate/up partial sums (64 rows x 98304 outputs in
    float32) and the down projection's partial sums need more than the 32 MiB
    array: refused with UNSUPPORTED before anything runs (lengths unchanged);
    a batch of 8 on the same model fits and equals ee_decode_step.  At the 8B
    widths (F 14336) a batch of 16 fits and equals ee_decode_step."""
    from kv_shared_exit_amd import _binding as Bd

    def run(sh, seed, refuse):
        w = synth.make_weights(sh, seed)
        dev = api.upload_weights(w)
        del w
        m = api.Model(sh, dev, gamma=2.0, max_batch=16, max_positions=8)
        ref, sta = api.KVCache(m, 16, 8), api.KVCache(m, 16, 8)
        try:
            prompts = np.random.default_rng(seed).integers(0, sh.vocab, (16, 3)).astype(np.int32)
            t0 = api.prefill(m, ref, prompts)
            api.prefill(m, sta, prompts)
            if refuse:
                with pytest.raises(Bd.EEError) as e:
                    api.decode_step_static(m, sta, 16, tokens=t0)
                assert e.value.status == Bd.EE_ERR_UNSUPPORTED
                assert list(sta.lengths()) == [3] * 16
            else:
                tr, er = api.decode_step(m, ref, 16, tokens=t0)
                ts, es = api.decode_step_static(m, sta, 16, tokens=t0)
                np.testing.assert_array_equal(ts, tr)
                np.testing.assert_array_equal(es, er)
                t0 = tr
            tr, er = api.decode_step(m, ref, 8, tokens=t0[:8])
            ts, es = api.decode_step_static(m, sta, 8, tokens=t0[:8])
            np.testing.assert_array_equal(ts, tr)
            np.testing.assert_array_equal(es, er)
        finally:
            ref.close()
            sta.close()
            m.close()

    run(ModelShape(1, 4096, 32, 8, 128, 49152, 1000, 128, rope_theta=500000.0), 23, True)
    run(ModelShape(1, 4096, 32, 8, 128, 14336, 1000, 128, rope_theta=500000.0), 22, False)
