"""Python front end of libee: device weights, models, KV caches, prefill and decode steps.

This layer marshals arguments only: PyTorch provides device memory and the HIP
stream; every step of the decode path runs in libee's kernels.  The function
names follow the C ABI (ee_create_model, ee_prefill, ee_decode_step,
ee_kv_cache_*).
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _binding as B

LINEAR = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
WHICH = {n: i for i, n in enumerate(LINEAR)}


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("libee needs a ROCm GPU (torch.cuda.is_available() is False)")
    return torch


def upload_weights(w: dict, device="cuda") -> dict:
    """Copy synth-style weights (uint16 bf16 bit patterns) to device tensors (int16 storage)."""
    torch = _torch()

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)

    out = {"tok_emb": up(w["tok_emb"]), "lm_head": up(w["lm_head"]),
           "final_norm": up(w["final_norm"]), "layers": []}
    for lw in w["layers"]:
        out["layers"].append({k: up(v) for k, v in lw.items()})
    return out


class Model:
    """ee_create_model over device weights (kept referenced for the model's lifetime)."""

    def __init__(self, shape, dev_weights: dict, gamma=None, exit_mode: int = B.EE_EXIT_INT4,
                 max_batch: int = 8, max_positions: int = 4096, criterion: int = B.EE_CRIT_HEAD,
                 check_every: int = 1, exit_rule: int = B.EE_RULE_SEQUENCE, temperature: float = 0.0,
                 sample_seed: int = 0, prefill_exit: bool = False):
        self.lib = B.load()
        self.shape = shape
        self.w = dev_weights
        L = shape.n_layers
        cfg = B.ModelConfig(L, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                            shape.d_ff, shape.vocab, shape.group, shape.rms_eps, shape.rope_theta,
                            exit_mode, max_batch, max_positions, criterion, check_every, exit_rule,
                            float(temperature), int(sample_seed), int(bool(prefill_exit)))
        layers = (B.LayerWeights * L)()
        for i, lw in enumerate(dev_weights["layers"]):
            for name in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down"):
                setattr(layers[i], name, lw[name].data_ptr())
            layers[i].head_T = lw["head_T"].data_ptr() if "head_T" in lw else None
        wts = B.Weights(dev_weights["tok_emb"].data_ptr(), dev_weights["lm_head"].data_ptr(),
                        dev_weights["final_norm"].data_ptr(), layers)
        self._layers = layers
        g = None
        if gamma is not None:
            g = np.ascontiguousarray(np.broadcast_to(np.asarray(gamma, np.float32), (L - 1,)))
        self._gamma = g
        h = C.c_void_p()
        B.check(self.lib.ee_create_model(C.byref(cfg), C.byref(wts), B._ptr(g), C.byref(h)))
        self.h = h
        self.cfg = cfg
        self.exit_mode = exit_mode

    def close(self):
        if self.h:
            B.check(self.lib.ee_destroy_model(self.h))
            self.h = None

    def exit_weights(self, layer: int, name: str, row0: int = 0, nrows: int | None = None):
        """(codes int8 [nrows, K], scales uint16 [nrows, K/G]) of an int4 exit copy."""
        sh = self.shape
        N, K = sh.linear_shapes()[name]
        nrows = N - row0 if nrows is None else nrows
        codes = np.empty((nrows, K), np.int8)
        scales = np.empty((nrows, K // sh.group), np.uint16)
        B.check(self.lib.ee_exit_weights_read(self.h, layer, WHICH[name], row0, nrows,
                                              B._ptr(codes), B._ptr(scales)))
        return codes, scales

    def profile(self, on: bool):
        B.check(self.lib.ee_profile_enable(self.h, int(on)))

    def profile_read(self, kind: int = 0):
        n = C.c_int64()
        ms = C.c_double()
        B.check(self.lib.ee_profile_read(self.h, kind, C.byref(n), C.byref(ms)))
        return n.value, ms.value


class KVCache:
    """ee_kv_cache_* over a library-owned or caller-owned device buffer."""

    def __init__(self, model: Model, max_batch: int, max_seq: int, track: bool = False,
                 torch_buffer: bool = True):
        self.model = model
        self.lib = model.lib
        self.max_batch, self.max_seq = max_batch, max_seq
        nbytes = C.c_size_t()
        B.check(self.lib.ee_kv_cache_bytes(model.h, max_batch, max_seq, C.byref(nbytes)))
        self.buf = None
        ptr = None
        if torch_buffer:
            torch = _torch()
            self.buf = torch.empty(nbytes.value, dtype=torch.uint8, device="cuda")
            ptr = self.buf.data_ptr()
        h = C.c_void_p()
        flags = B.EE_KV_TRACK_OCCUPANCY if track else 0
        B.check(self.lib.ee_kv_cache_create(model.h, max_batch, max_seq, ptr, nbytes.value, flags,
                                            C.byref(h)))
        self.h = h

    def close(self):
        if self.h:
            B.check(self.lib.ee_kv_cache_destroy(self.h))
            self.h = None

    def reset(self, seq: int = -1):
        B.check(self.lib.ee_kv_cache_reset(self.h, seq))

    def rollback(self, seq: int = -1, n: int = 1):
        B.check(self.lib.ee_kv_cache_rollback(self.h, seq, n))

    def lengths(self) -> np.ndarray:
        out = np.empty(self.max_batch, np.int32)
        B.check(self.lib.ee_kv_cache_lengths(self.h, B._ptr(out)))
        return out

    def read(self, layer: int, seq: int, pos0: int, n: int):
        """(K, V) bf16 bit patterns [n, Hkv, hd] of one layer (1-based) and sequence."""
        sh = self.model.shape
        k = np.empty((n, sh.n_kv_heads, sh.head_dim), np.uint16)
        v = np.empty_like(k)
        B.check(self.lib.ee_kv_cache_read(self.h, layer, seq, pos0, n, B._ptr(k), B._ptr(v)))
        return k, v

    def occupancy(self) -> np.ndarray:
        sh = self.model.shape
        out = np.empty((sh.n_layers, self.max_batch, self.max_seq), np.uint8)
        B.check(self.lib.ee_kv_cache_occupancy(self.h, B._ptr(out)))
        return out


def _stream_ptr(stream):
    if stream is None:
        return None
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def prefill(model: Model, cache: KVCache, prompts, stream=None, logits: bool = False, exits: bool = False):
    """Prefill; returns the first tokens, plus the last position's logits with
    ``logits`` and each sequence's prefill exit layer with ``exits`` (in that
    order, as a tuple when either is asked for)."""
    prompts = np.ascontiguousarray(prompts, dtype=np.int32)
    batch, P = prompts.shape
    out = np.empty(batch, np.int32)
    lg = np.empty((batch, model.shape.vocab), np.float32) if logits else None
    ex = np.empty(batch, np.int32) if exits else None
    B.check(model.lib.ee_prefill(model.h, cache.h, batch, B._ptr(prompts), P,
                                 _stream_ptr(stream), B._ptr(out), B._ptr(lg), B._ptr(ex)))
    res = (out,) + ((lg,) if logits else ()) + ((ex,) if exits else ())
    return res if len(res) > 1 else out


def decode_step(model: Model, cache: KVCache, batch: int, tokens=None, forced=None, gamma=None,
                stream=None, debug: dict | None = None):
    """One decode step.  ``debug`` may name the outputs to return ("p", "logits",
    "hidden", "gap") as a dict of None placeholders; they are filled in place."""
    sh = model.shape
    L = sh.n_layers
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    frc = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32)
    gam = None
    if gamma is not None:
        gam = np.ascontiguousarray(np.broadcast_to(np.asarray(gamma, np.float32), (L - 1,)))
    out_t = np.empty(batch, np.int32)
    out_e = np.empty(batch, np.int32)
    dbg_ptr = None
    if debug is not None:
        if "p" in debug:
            debug["p"] = np.empty((batch, max(L - 1, 1)), np.float32)
        if "logits" in debug:
            debug["logits"] = np.empty((batch, sh.vocab), np.float32)
        if "hidden" in debug:
            debug["hidden"] = np.empty((batch, L + 1, sh.d_model), np.float32)
        if "gap" in debug:
            debug["gap"] = np.empty(batch, np.float32)
        dbg = B.StepDebug(B._ptr(debug.get("p")), B._ptr(debug.get("logits")),
                          B._ptr(debug.get("hidden")), B._ptr(debug.get("gap")))
        dbg_ptr = C.byref(dbg)
    B.check(model.lib.ee_decode_step(model.h, cache.h, batch, B._ptr(tok), B._ptr(frc),
                                     B._ptr(gam), _stream_ptr(stream), B._ptr(out_t),
                                     B._ptr(out_e), dbg_ptr))
    return out_t, out_e


def decode_step_static(model: Model, cache: KVCache, batch: int, tokens=None, forced=None, gamma=None,
                       stream=None):
    """ee_decode_step_static: the decode step with its workspaces in the
    library's static device array (no allocation); same results as
    decode_step without diagnostics."""
    L = model.shape.n_layers
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    frc = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32)
    gam = None
    if gamma is not None:
        gam = np.ascontiguousarray(np.broadcast_to(np.asarray(gamma, np.float32), (L - 1,)))
    out_t = np.empty(batch, np.int32)
    out_e = np.empty(batch, np.int32)
    B.check(model.lib.ee_decode_step_static(model.h, cache.h, batch, B._ptr(tok), B._ptr(frc), B._ptr(gam),
                                            _stream_ptr(stream), B._ptr(out_t), B._ptr(out_e)))
    return out_t, out_e
