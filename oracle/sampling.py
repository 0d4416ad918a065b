"""Sampled decoding with AdaDecode's verification of the early draft.

TEST INFRASTRUCTURE: part of the CPU oracle.  Only tests/, the smoke check and
bench.py's cpu_baseline leg may import it; the product path never does.

AdaDecode explainer, section 3.1 (verification): a token predicted early (the
draft, from the intermediate layer's distribution) is accepted with
probability min(1, p_final / p_draft) of that token; if it is rejected, the
token is drawn from the normalised relu(p_final - p_draft).  Section 2.2 makes
the draft at the layer where the exit head's confidence passes the threshold.
Reading (the pages print only the greedy case's building blocks and this
routine): with temperature tau, p_draft = softmax(exit-head logits / tau) at the
sequence's exit layer and p_final = softmax(final logits / tau); a sequence
that does not exit (e = L) has no draft and draws from p_final.  The exit
decision itself is unchanged (top-1 probability of the exit head at
temperature 1 against gamma).

Random numbers are drawn from a counter-based generator so that the GPU path
can draw the same ones: Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC 2011), key (seed, 0),
counter (v // 4, sequence, position, stream), word v % 4 for vocabulary entry
v.  A 64-bit word x gives the uniform u = ((x >> 41) + 0.5) / 2^23 in (0, 1)
(24 significant bits: exact in float32).  Categorical draws use the Gumbel-max rule: argmax over v
of score_v + G_v with G = -log(-log(u)) (lowest index on ties), which draws v
with probability proportional to exp(score_v).  The acceptance test uses word
0 of the block with counter (0, sequence, position, STREAM_ACCEPT).
"""
from __future__ import annotations

import numpy as np

STREAM_DRAFT = 1      # the draft from the exit head's distribution
STREAM_FINAL = 2      # a sequence without a draft, from the final distribution
STREAM_RESAMPLE = 3   # after a rejection, from relu(p_final - p_draft)
STREAM_ACCEPT = 4     # the acceptance uniform

_M32 = np.uint64(0xFFFFFFFF)
_MUL = (np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157))
_WEYL = (np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B))


def _mulhilo(a, m):
    """(high, low) 64-bit halves of the 128-bit product a * m (a: uint64 array)."""
    a = np.asarray(a, np.uint64)
    al, ah = a & _M32, a >> np.uint64(32)
    ml, mh = m & _M32, m >> np.uint64(32)
    with np.errstate(over="ignore"):
        p0, p1, p2, p3 = al * ml, al * mh, ah * ml, ah * mh
        mid = (p0 >> np.uint64(32)) + (p1 & _M32) + (p2 & _M32)
        hi = p3 + (p1 >> np.uint64(32)) + (p2 >> np.uint64(32)) + (mid >> np.uint64(32))
        lo = a * m
    return hi, lo


def philox4x64(counter, key, rounds: int = 10):
    """The Philox4x64 block function: counter = 4 uint64 arrays (broadcast),
    key = 2 uint64 integers; returns the 4 output words."""
    x0, x1, x2, x3 = [np.asarray(c, np.uint64) for c in counter]
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    for r in range(rounds):
        if r:
            with np.errstate(over="ignore"):
                k0, k1 = k0 + _WEYL[0], k1 + _WEYL[1]
        hi0, lo0 = _mulhilo(x0, _MUL[0])
        hi1, lo1 = _mulhilo(x2, _MUL[1])
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def uniforms(seed: int, pos: int, seq: int, stream: int, n: int) -> np.ndarray:
    """u_v for v = 0..n-1 (float64 holding float32-exact values in (0, 1))."""
    blocks = np.arange((n + 3) // 4, dtype=np.uint64)
    w = philox4x64((blocks, np.uint64(seq), np.uint64(pos), np.uint64(stream)), (seed, 0))
    x = np.stack(w, axis=1).reshape(-1)[:n]
    return ((x >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel(seed: int, pos: int, seq: int, stream: int, n: int) -> np.ndarray:
    return -np.log(-np.log(uniforms(seed, pos, seq, stream, n)))


def gumbel_argmax(scores: np.ndarray, g: np.ndarray):
    """(index, margin): argmax of scores + g (lowest index on ties) and the gap
    to the second-best perturbed score (inf with one finite candidate)."""
    s = np.asarray(scores, np.float64) + g
    i = int(np.argmax(s))
    fin = np.sort(s[np.isfinite(s)])
    margin = float(fin[-1] - fin[-2]) if fin.size > 1 else np.inf
    return i, margin


def softmax_t(logits: np.ndarray, tau: float) -> np.ndarray:
    z = np.asarray(logits, np.float64) / tau
    z = z - z.max()
    p = np.exp(z)
    return p / p.sum()


def sample_token(final_logits, exit_logits, tau: float, seed: int, pos: int, seq: int):
    """The emitted token of one sequence and the decisions behind it.

    exit_logits is None for a sequence that did not exit (no draft).  Returns
    (token, info) with info: draft, accepted (None without a draft), and the
    margins of every decision taken (perturbed top-2 gaps; for the acceptance,
    |u p_draft - p_final| relative to max(p_draft, p_final)), which the parity
    tests use to skip near ties."""
    V = len(final_logits)
    pf = softmax_t(final_logits, tau)
    if exit_logits is None:
        tok, m = gumbel_argmax(np.asarray(final_logits, np.float64) / tau,
                               gumbel(seed, pos, seq, STREAM_FINAL, V))
        return tok, {"draft": None, "accepted": None, "margins": [m]}
    pd = softmax_t(exit_logits, tau)
    draft, m1 = gumbel_argmax(np.asarray(exit_logits, np.float64) / tau,
                              gumbel(seed, pos, seq, STREAM_DRAFT, V))
    u = uniforms(seed, pos, seq, STREAM_ACCEPT, 1)[0]
    # accept with probability min(1, p_final / p_draft): u < p_final / p_draft
    lhs, rhs = u * pd[draft], pf[draft]
    m2 = abs(lhs - rhs) / max(pd[draft], pf[draft])
    if lhs < rhs:
        return draft, {"draft": draft, "accepted": True, "margins": [m1, m2]}
    r = np.maximum(pf - pd, 0.0)
    with np.errstate(divide="ignore"):
        score = np.where(r > 0, np.log(r), -np.inf)
    tok, m3 = gumbel_argmax(score, gumbel(seed, pos, seq, STREAM_RESAMPLE, V))
    return tok, {"draft": draft, "accepted": False, "margins": [m1, m2, m3]}
