"""Seeded synthetic inputs for the KV-shared early-exit decode step.

This module is shared by the CPU oracle and by the HIP path, and it is the only
code they share.  It holds workload shapes, seeded random weights (bf16 bit
patterns), prompts, forced-exit schedules and the target exit-layer
distribution.  It holds none of the decode method's arithmetic: no norm, no
projection, no attention, no exit head, no quantiser.

Weights follow the random-init recipe of the workloads: every linear matrix is
drawn N(0, 0.02^2) in float32 and rounded to bf16 (round to nearest, ties to
even); norm gains are 1.  The exit-head matrix T of layer l is drawn with
standard deviation 0.02 * alpha_l, where alpha_l is a per-layer logit scale
chosen by calibration so that the exit layers follow a target distribution
(stored under ``synth/calibration/``; missing file means alpha_l = 1).

Layouts (all row-major, ``[out, in]`` for linear maps):
    tok_emb [V, d], lm_head [V, d], final_norm [d]
    per layer: attn_norm [d], wq [H*hd, d], wk [Hkv*hd, d], wv [Hkv*hd, d],
               wo [d, H*hd], ffn_norm [d], w_gate [F, d], w_up [F, d],
               w_down [d, F], head_T [d, d] (layers 1..L-1 only; output j of
               the head projection is row j, i.e. z_j = sum_i T[j, i] h_i).
"""
from __future__ import annotations

import json
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "ModelShape", "Workload", "WORKLOADS", "workload", "make_weights",
    "make_prompts", "make_forced_exits", "make_target_exits", "geometric_hazard", "exit_pmf",
    "load_alpha", "load_tau", "layer_names", "bf16_bits_to_f32",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
CALIB_DIR = os.path.join(_HERE, "calibration")


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    group: int                 # int4 group size along the input dimension
    rms_eps: float = 1e-5
    rope_theta: float = 1.0e4

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def linear_shapes(self) -> dict:
        d, F = self.d_model, self.d_ff
        return {"wq": (self.q_dim, d), "wk": (self.kv_dim, d), "wv": (self.kv_dim, d),
                "wo": (d, self.q_dim), "w_gate": (F, d), "w_up": (F, d), "w_down": (d, F)}

    def params_per_layer(self) -> int:
        return sum(a * b for a, b in self.linear_shapes().values())


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    batch: int
    prompt_len: int
    gen_tokens: int            # generated tokens, the prefill's first token included
    gamma: float               # exit threshold (same for every layer)
    policy: str                # "calibrated" | "forced"
    mean_exit: float | None    # target mean exit layer (calibrated policy)
    forced_lo: int = 0         # forced policy: exit layer uniform in [lo, hi]
    forced_hi: int = 0
    index: int = 0             # seeds: weights 0+i, prompts 1000+i, calib 2000+i, forced 3000+i

    @property
    def seed_weights(self) -> int:
        return self.index

    @property
    def seed_prompts(self) -> int:
        return 1000 + self.index

    @property
    def seed_calib(self) -> int:
        return 2000 + self.index

    @property
    def seed_forced(self) -> int:
        return 3000 + self.index

    @property
    def decode_steps(self) -> int:
        return self.gen_tokens - 1


TINY = ModelShape(4, 128, 4, 4, 32, 512, 1024, 32, rope_theta=1.0e4)
LLAMA1B = ModelShape(16, 2048, 32, 8, 64, 8192, 128256, 128, rope_theta=5.0e5)
LLAMA8B = ModelShape(32, 4096, 32, 8, 128, 14336, 128256, 128, rope_theta=5.0e5)
CODELLAMA34B = ModelShape(48, 8192, 64, 8, 128, 22016, 32000, 128, rope_theta=1.0e6)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, 1, 16, 32, 0.75, "calibrated", 1.5, index=0),
    "1b": Workload("1b", LLAMA1B, 1, 512, 256, 0.75, "calibrated", 4.81, index=1),
    "8b": Workload("8b", LLAMA8B, 8, 1024, 256, 0.75, "calibrated", 16.0, index=2),
    "8b_b64": Workload("8b_b64", LLAMA8B, 64, 4096, 128, 0.75, "forced", None, 8, 32, index=3),
    "34b": Workload("34b", CODELLAMA34B, 4, 2048, 256, 0.85, "calibrated", 30.0, index=4),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def layer_names(shape: ModelShape, layer: int) -> list:
    """Names of the tensors of 1-based layer ``layer``."""
    names = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down"]
    if layer < shape.n_layers:
        names.append("head_T")
    return names


# ----------------------------------------------------------------------------
# seeded bf16 draws
# ----------------------------------------------------------------------------
_CHUNK = 1 << 22
_KIND = {"tok_emb": 1, "lm_head": 2, "final_norm": 3, "attn_norm": 10, "wq": 11, "wk": 12,
         "wv": 13, "wo": 14, "ffn_norm": 15, "w_gate": 16, "w_up": 17, "w_down": 18,
         "head_T": 19}


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the uint16 bit pattern.

    Inputs here are finite normal draws, so no NaN handling is needed.
    """
    u = a.view(np.uint32)
    u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _tensor_id(name: str, layer: int) -> int:
    return _KIND[name] * 4096 + layer


def _normal_chunk(seed: int, tid: int, chunk: int, n: int) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, chunk])
    return rng.standard_normal(n, dtype=np.float32)


def _draw_bf16(seed: int, tid: int, shape, std: float, pool=None) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + _CHUNK - 1) // _CHUNK
    s32 = np.float32(std)

    def work(c):
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        z = _normal_chunk(seed, tid, c, hi - lo)
        z *= s32
        out[lo:hi] = _f32_to_bf16_bits(z)

    if pool is None or nchunks == 1:
        for c in range(nchunks):
            work(c)
    else:
        list(pool.map(work, range(nchunks)))
    return out.reshape(shape)


def draw_unit_normal(seed: int, name: str, layer: int, shape) -> np.ndarray:
    """The float32 standard-normal draws behind a tensor (before scaling and rounding)."""
    n = int(np.prod(shape))
    tid = _tensor_id(name, layer)
    parts = []
    for c in range((n + _CHUNK - 1) // _CHUNK):
        lo = c * _CHUNK
        parts.append(_normal_chunk(seed, tid, c, min(n, lo + _CHUNK) - lo))
    return np.concatenate(parts).reshape(shape)


def load_alpha(wl: Workload) -> np.ndarray | None:
    """Per-layer exit-head scales alpha_l (l = 1..L-1) for a workload, or None."""
    path = os.path.join(CALIB_DIR, f"{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    alpha = np.asarray(data["alpha"], dtype=np.float64)
    assert alpha.shape == (wl.shape.n_layers - 1,)
    return alpha


def load_tau(wl: Workload, batch_min: bool = False) -> np.ndarray | None:
    """Per-layer similarity thresholds tau_l (l = 1..L-1) of a workload's state
    transition similarity criterion (for the batch-minimum rule with
    ``batch_min``), or None."""
    path = os.path.join(CALIB_DIR, f"{wl.name}_sts.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    key = "tau_batch_min" if batch_min else "tau"
    if key not in data:
        return None
    tau = np.asarray(data[key], dtype=np.float64)
    assert tau.shape == (wl.shape.n_layers - 1,)
    return tau


def make_weights(shape: ModelShape, seed: int, alpha=None, threads: int | None = None,
                 layers=None) -> dict:
    """Seeded bf16 weights as uint16 bit patterns.

    Returns ``{"tok_emb", "lm_head", "final_norm", "layers": [dict per layer]}``.
    ``alpha`` is the per-layer exit-head scale (length L-1, default all ones).
    ``layers`` optionally restricts which 1-based layers are drawn (others None).
    """
    L, d = shape.n_layers, shape.d_model
    if alpha is None:
        alpha = np.ones(L - 1)
    threads = threads or min(16, os.cpu_count() or 1)
    one = np.full(d, 0x3F80, dtype=np.uint16)          # bf16(1.0)
    with ThreadPoolExecutor(threads) as pool:
        w = {
            "tok_emb": _draw_bf16(seed, _tensor_id("tok_emb", 0), (shape.vocab, d), 0.02, pool),
            "lm_head": _draw_bf16(seed, _tensor_id("lm_head", 0), (shape.vocab, d), 0.02, pool),
            "final_norm": one.copy(),
            "layers": [],
        }
        for l in range(1, L + 1):
            if layers is not None and l not in layers:
                w["layers"].append(None)
                continue
            lw = {"attn_norm": one.copy(), "ffn_norm": one.copy()}
            for name, shp in shape.linear_shapes().items():
                lw[name] = _draw_bf16(seed, _tensor_id(name, l), shp, 0.02, pool)
            if l < L:
                lw["head_T"] = _draw_bf16(seed, _tensor_id("head_T", l), (d, d),
                                          0.02 * float(alpha[l - 1]), pool)
            w["layers"].append(lw)
    return w


def make_prompts(wl: Workload, batch: int | None = None, length: int | None = None,
                 seed: int | None = None) -> np.ndarray:
    """Uniform random token ids, int32 [batch, length]."""
    batch = wl.batch if batch is None else batch
    length = wl.prompt_len if length is None else length
    seed = wl.seed_prompts if seed is None else seed
    rng = np.random.default_rng([seed, 0])
    return rng.integers(0, wl.shape.vocab, size=(batch, length), dtype=np.int64).astype(np.int32)


def make_forced_exits(wl: Workload, step: int, batch: int | None = None,
                      lo: int | None = None, hi: int | None = None) -> np.ndarray:
    """Forced exit layers for one decode step, int32 [batch], uniform in [lo, hi]."""
    batch = wl.batch if batch is None else batch
    lo = wl.forced_lo if lo is None else lo
    hi = wl.forced_hi if hi is None else hi
    rng = np.random.default_rng([wl.seed_forced, step])
    return rng.integers(lo, hi + 1, size=batch, dtype=np.int64).astype(np.int32)


def make_target_exits(wl: Workload, step: int, batch: int | None = None) -> np.ndarray:
    """Exit layers for one decode step drawn from a calibrated workload's
    target distribution (truncated geometric with the workload's mean exit
    layer), int32 [batch].  Used as forced exits where no calibrated exit-head
    scales exist, so that the step runs the exit layers the calibration aims
    at; seeded like the forced schedules (a second stream of the same seed)."""
    assert wl.mean_exit is not None
    batch = wl.batch if batch is None else batch
    L = wl.shape.n_layers
    cdf = np.cumsum(exit_pmf(geometric_hazard(wl.mean_exit, L), L))
    u = np.random.default_rng([wl.seed_forced, 1, step]).random(batch)
    return (np.searchsorted(cdf, u * cdf[-1], side="right") + 1).clip(1, L).astype(np.int32)


def exit_pmf(h: float, L: int) -> np.ndarray:
    """Truncated-geometric exit-layer distribution over e = 1..L with hazard h."""
    e = np.arange(1, L + 1, dtype=np.float64)
    pmf = h * (1.0 - h) ** (e - 1)
    pmf[-1] = (1.0 - h) ** (L - 1)
    return pmf


def geometric_hazard(mean_exit: float, L: int) -> float:
    """Constant per-layer hazard whose truncated-geometric exit layer has the given mean."""
    lo, hi = 0.0, 1.0
    e = np.arange(1, L + 1, dtype=np.float64)
    for _ in range(200):
        m = 0.5 * (lo + hi)
        if float((exit_pmf(m, L) * e).sum()) > mean_exit:
            lo = m
        else:
            hi = m
    return 0.5 * (lo + hi)
