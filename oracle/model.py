"""Oracle decoder, exit heads, exit river and shared KV cache (test infrastructure).

What one decode step computes, per sequence b (decisions are per token and per
layer: CALM explainer section 2.2; AdaDecode explainer section 2.2), with
layers numbered l = 1..L and exit layer e in 1..L (e = L: no exit):

  h = E_in[token]                                   embedding row, exact
  for l = 1..L:
      weights = backbone layer l        if the sequence has not exited
              = int4 exit copy of l     otherwise   (River-LLM section 4.1-4.2)
      x = bf16(rmsnorm(h) * g_attn)
      q, k, v = bf16(Wq x), bf16(Wk x), bf16(Wv x)
      q, k = bf16(rope(q, pos)), bf16(rope(k, pos))
      K_l[pos], V_l[pos] = k, v          one shared slot per (layer, position),
                                          whichever copy produced it
                                          (River-LLM sections 4.3 and 8.2)
      o_i = bf16(softmax(q_i K_j^T / sqrt(hd)) V_j), j = kv head of q head i
                                          (River-LLM section 3.1; grouped heads)
      h = h + Wo o
      x = bf16(rmsnorm(h) * g_ffn)
      a = bf16(silu(Wg x) * (Wu x));  h = h + Wd a
      if not exited and l < L:            exit head (AdaDecode section 2.1)
          z = bf16(T_l bf16(h));  logits = E z;  p = max softmax(logits)
          exit iff p > gamma_l  (strict; AdaDecode section 2.2)  -> e = l
  token = argmax(E_out bf16(rmsnorm(h) * g_final)), lowest index on ties

With criterion "sts" the exit head is replaced by River-LLM's state
transition similarity (River-LLM explainer, sections 5.1-5.2): after layer l
the cosine between the row's hidden state entering the layer and leaving it
(each normalised to unit length, then the dot product, float64), and the row
exits iff that similarity > tau_l (the per-layer thresholds take gamma's
place).  The pages apply the threshold to the batch minimum; here, as for the
exit head, each sequence decides for itself.

With exit_rule "batch_min" (River-LLM explainer, section 5.2: the exit fires
when the minimum over the batch's tokens exceeds the threshold) the sequences
on the backbone whose exit is not forced leave together after the first
evaluated layer at which the smallest of their values > the threshold.

With check_every = N > 1 the criterion is evaluated only after layers N, 2N,
... (CALM explainer's check every N layers; AdaDecode's layer subsets); after
the other layers no sequence exits unless its exit is forced there.

The token of a step is the greedy argmax of the final LM head after the exit
river has finished the remaining layers; the exit head only decides which
copy runs the remaining layers (the reading under which "unquantised exit
layers give full-depth decoding" holds).

Prefill runs every prompt position at full depth with the backbone weights
(no exit heads), writes every KV slot and returns the greedy token after the
last position (River-LLM section 6.1 names the two phases; the prefill exit
rule is not specified, so prefill does not exit).

RMSNorm uses epsilon from the model shape and mean(h^2) over the hidden
dimension; RoPE rotates pairs (i, i + hd/2) by pos * theta^(-2i/hd) with a
cos/sin table computed in float64 and rounded to float32; silu(g) = g/(1+e^-g).

Pins (``tests/test_oracle_*.py``): attention, RMSNorm, SiLU, RoPE and softmax
against torch CPU library routines and closed forms; the exit head against
closed forms (identity and permutation heads over a diagonal E, inputs placed
off the bf16 grid so that each of its two roundings shows, T = 0 giving 1/V,
no dependence on the final norm's gain, E and not the input embedding); gamma > 1 equals a plain
decoder written from torch library calls; gamma <= 0 equals a plain decoder
whose layers 2..L are the dequantised copies; unquantised exit copies equal
full depth for any schedule; every KV slot is written exactly once; a sequence
alone equals the same sequence inside a batch; token-by-token prefill equals
the layer-major prefill.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round, from_bf16_bits, f32_round
from .quant import quantize_int4, dequantize_int4
from .sampling import sample_token

LINEAR = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


# ----------------------------------------------------------------------------
# elementary operations
# ----------------------------------------------------------------------------
def rmsnorm(h: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """bf16(h / sqrt(mean(h^2) + eps) * g) over the last axis."""
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return bf16_round(h / np.sqrt(ms + eps) * g)


def rope_table(n_pos: int, head_dim: int, theta: float):
    """cos and sin of pos * theta^(-2i/hd), i < hd/2, computed in float64 then rounded to float32."""
    half = head_dim // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return f32_round(np.cos(ang)), f32_round(np.sin(ang))


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on the last axis; cos/sin broadcast over heads."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return bf16_round(np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1))


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def softmax_top1(logits: np.ndarray) -> np.ndarray:
    """max_v softmax(logits)_v = 1 / sum_v exp(l_v - max l), over the last axis."""
    m = logits.max(axis=-1, keepdims=True)
    return 1.0 / np.exp(logits - m).sum(axis=-1)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, n_kv_heads: int) -> np.ndarray:
    """Decode attention of one position.

    q [H, hd]; K, V [Hkv, T, hd] (all keys visible).  q head i reads kv head
    i // (H / Hkv).  Returns bf16 o [H * hd].
    """
    H, hd = q.shape
    group = H // n_kv_heads
    out = np.empty((H, hd))
    scale = 1.0 / np.sqrt(hd)
    for i in range(H):
        j = i // group
        s = (K[j] @ q[i]) * scale
        pi = np.exp(s - s.max())
        pi /= pi.sum()
        out[i] = pi @ V[j]
    return bf16_round(out.reshape(-1))


def lin(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """x @ W^T for a linear map stored [out, in], in W's precision, returned as float64."""
    if W.dtype == np.float64:
        return x @ W.T
    return (x.astype(W.dtype) @ W.T).astype(np.float64)


# ----------------------------------------------------------------------------
# model and shared KV cache
# ----------------------------------------------------------------------------
class OracleModel:
    """Weights of the decoder, its exit heads and its int4 exit copies.

    ``weights`` is the dict produced by ``synth.make_weights`` (bf16 bit
    patterns).  ``exit_mode`` is "int4" (exit copies are the quantised layers)
    or "bf16" (exit copies are the backbone layers themselves).  ``cache_f64``
    keeps widened copies of every matrix (fast, memory hungry); otherwise each
    matrix is widened when used.  ``matmul_dtype`` is float64 for every
    comparison made by the tests; the exit-head calibration, which only picks
    inputs, may ask for float32 matrix products to reach the 8B shape.
    """

    def __init__(self, shape, weights, exit_mode: str = "int4", cache_f64: bool = True,
                 matmul_dtype=np.float64):
        if exit_mode not in ("int4", "bf16"):
            raise ValueError(exit_mode)
        self.shape = shape
        self.raw = weights
        self.exit_mode = exit_mode
        self.cache_f64 = cache_f64
        self.mdt = np.dtype(matmul_dtype)
        self._f64 = {}
        self._q = {}
        self.tok_emb = from_bf16_bits(weights["tok_emb"])
        self.lm_head = from_bf16_bits(weights["lm_head"])
        self.final_norm = from_bf16_bits(weights["final_norm"])
        self.cos, self.sin = None, None

    # -- weights -----------------------------------------------------------
    def w(self, layer: int, name: str) -> np.ndarray:
        """Backbone tensor of 1-based ``layer`` as float64."""
        key = (layer, name)
        if key in self._f64:
            return self._f64[key]
        t = from_bf16_bits(self.raw["layers"][layer - 1][name])
        if t.ndim == 2 and self.mdt != np.float64:
            t = t.astype(self.mdt)
        if self.cache_f64:
            self._f64[key] = t
        return t

    def quantized(self, layer: int, name: str):
        """(codes int8 [N, K], scales float64 [N, K/G]) of the exit copy of a linear map."""
        key = (layer, name)
        if key not in self._q:
            self._q[key] = quantize_int4(from_bf16_bits(self.raw["layers"][layer - 1][name]),
                                         self.shape.group)
        return self._q[key]

    def w_exit(self, layer: int, name: str) -> np.ndarray:
        """Exit-copy matrix of a linear map as float64 (dequantised int4, or the backbone)."""
        if self.exit_mode == "bf16":
            return self.w(layer, name)
        key = (layer, name, "exit")
        if key in self._f64:
            return self._f64[key]
        q, s = self.quantized(layer, name)
        t = dequantize_int4(q, s, self.shape.group).astype(self.mdt)
        if self.cache_f64:
            self._f64[key] = t
        return t

    def rope(self, n_pos: int):
        if self.cos is None or self.cos.shape[0] < n_pos:
            self.cos, self.sin = rope_table(max(n_pos, 16), self.shape.head_dim,
                                            self.shape.rope_theta)
        return self.cos, self.sin


class KVCache:
    """Shared K/V store: one slot per (layer, sequence, position).

    Entries are bf16 values held in float32.  ``occ`` counts the writes of
    each slot (River-LLM section 8.2 stores every layer's K/V whether a
    backbone layer or an exit layer produced it).
    """

    def __init__(self, shape, batch: int, max_seq: int):
        L, Hkv, hd = shape.n_layers, shape.n_kv_heads, shape.head_dim
        self.shape = shape
        self.max_seq = max_seq
        self.K = np.zeros((L, batch, Hkv, max_seq, hd), dtype=np.float32)
        self.V = np.zeros_like(self.K)
        self.occ = np.zeros((L, batch, max_seq), dtype=np.int32)
        self.lens = np.zeros(batch, dtype=np.int64)

    def store(self, layer: int, b: int, pos: int, k: np.ndarray, v: np.ndarray):
        self.K[layer - 1, b, :, pos] = k
        self.V[layer - 1, b, :, pos] = v
        self.occ[layer - 1, b, pos] += 1

    def keys(self, layer: int, b: int, n: int):
        return (self.K[layer - 1, b, :, :n].astype(np.float64),
                self.V[layer - 1, b, :, :n].astype(np.float64))


# ----------------------------------------------------------------------------
# one layer for a group of rows that share one weight copy
# ----------------------------------------------------------------------------
def _layer_rows(model: OracleModel, cache: KVCache, layer: int, rows, h, pos, use_exit: bool):
    """Run layer ``layer`` for sequences ``rows`` in place on ``h`` (float64 [B, d])."""
    sh = model.shape
    H, Hkv, hd = sh.n_heads, sh.n_kv_heads, sh.head_dim
    W = model.w_exit if use_exit else model.w
    hr = h[rows]
    x = rmsnorm(hr, model.w(layer, "attn_norm"), sh.rms_eps)
    q = bf16_round(lin(x, W(layer, "wq"))).reshape(len(rows), H, hd)
    k = bf16_round(lin(x, W(layer, "wk"))).reshape(len(rows), Hkv, hd)
    v = bf16_round(lin(x, W(layer, "wv"))).reshape(len(rows), Hkv, hd)
    cos, sin = model.rope(int(max(pos[rows])) + 1)
    o = np.empty((len(rows), H * hd))
    for i, b in enumerate(rows):
        p = int(pos[b])
        qr = apply_rope(q[i], cos[p], sin[p])
        kr = apply_rope(k[i], cos[p], sin[p])
        cache.store(layer, b, p, kr, v[i])
        Kb, Vb = cache.keys(layer, b, p + 1)
        o[i] = attend(qr, Kb, Vb, Hkv)
    hr = hr + lin(o, W(layer, "wo"))
    x = rmsnorm(hr, model.w(layer, "ffn_norm"), sh.rms_eps)
    a = bf16_round(silu(lin(x, W(layer, "w_gate"))) * lin(x, W(layer, "w_up")))
    hr = hr + lin(a, W(layer, "w_down"))
    h[rows] = hr


def exit_head(model: OracleModel, layer: int, h: np.ndarray):
    """Exit head of ``layer`` on rows h [n, d]: (p_top1 [n], logits [n, V]).

    z = bf16(T_l bf16(h)); logits = E z with E the LM-head matrix
    (AdaDecode explainer section 2.1, head weight E T^(l)); p = max softmax.
    """
    z = bf16_round(lin(bf16_round(h), model.w(layer, "head_T")))
    logits = z @ model.lm_head.T
    return softmax_top1(logits), logits


def state_transition_similarity(h_in: np.ndarray, h_out: np.ndarray) -> np.ndarray:
    """Cosine similarity of a layer's input and output hidden states per row
    (River-LLM explainer, section 5.1): each row scaled to unit length (norm
    floored at 1e-12), then the dot product; float64."""
    a = np.asarray(h_in, dtype=np.float64)
    b = np.asarray(h_out, dtype=np.float64)
    na = np.maximum(np.sqrt((a * a).sum(axis=-1)), 1e-12)
    nb = np.maximum(np.sqrt((b * b).sum(axis=-1)), 1e-12)
    return ((a / na[..., None]) * (b / nb[..., None])).sum(axis=-1)


def final_head(model: OracleModel, h: np.ndarray):
    """Greedy token, top-2 logit gap and logits of the final LM head on rows h [n, d]."""
    y = rmsnorm(h, model.final_norm, model.shape.rms_eps)
    logits = y @ model.lm_head.T
    tok = np.argmax(logits, axis=-1)          # first maximum: lowest index on ties
    if logits.shape[-1] > 1:
        top2 = np.sort(logits, axis=-1)[:, -2:]
        gap = top2[:, 1] - top2[:, 0]
    else:
        gap = np.full(len(h), np.inf)
    return tok.astype(np.int32), gap, logits


# ----------------------------------------------------------------------------
# decode step, prefill, generation
# ----------------------------------------------------------------------------
def decode_step(model: OracleModel, cache: KVCache, tokens, gamma=None, forced=None,
                trace: bool = False, heads: bool = True, criterion: str = "head", check_every: int = 1,
                exit_rule: str = "sequence", temperature: float = 0.0, seed: int = 0):
    """One decode step for sequences 0..B-1 of ``cache`` (B = len(tokens)).

    ``gamma``: per-layer thresholds gamma_1..gamma_{L-1} (scalar broadcasts);
    with ``criterion="sts"`` they are the similarity thresholds tau_l.
    ``forced``: optional int [B]; 0 lets the criterion decide, 1..L forces the
    exit layer (the criterion is still evaluated; its decision is overridden).
    Returns ``(tokens [B], exit_layers [B], info)`` where info holds
    ``p`` [B, L-1] (the criterion's value: top-1 probability of the exit head,
    or the state transition similarity; NaN where not evaluated),
    ``head_absmax`` [B, L-1] (largest |logit| of each evaluated exit head),
    ``gap`` [B], ``logits`` [B, V] and, with ``trace``, ``hidden`` [B, L+1, d]
    (after the embedding and after every layer).  ``heads=False`` evaluates no
    criterion (no sequence exits); it is used to sample full-depth states.
    ``check_every``: the criterion runs after layers that are multiples of it;
    forced exits apply after any layer.  ``exit_rule``: "sequence" (each
    sequence decides for itself) or "batch_min" (the unforced sequences on the
    backbone exit together when the smallest of their values > the threshold).
    ``temperature`` > 0: sampled decoding with AdaDecode's verification
    (``oracle.sampling.sample_token``; the draft comes from the exit head's
    logits at the exit layer; needs the exit-head criterion checked after every
    layer); ``seed`` keys its counter-based generator.  info["sample"] then
    holds each row's decisions and their margins.
    """
    if criterion not in ("head", "sts"):
        raise ValueError(f"unknown criterion {criterion!r}")
    if exit_rule not in ("sequence", "batch_min"):
        raise ValueError(f"unknown exit rule {exit_rule!r}")
    if check_every < 1:
        raise ValueError("check_every must be >= 1")
    sampled = temperature > 0
    if sampled and (criterion != "head" or check_every != 1):
        raise ValueError("sampled decoding drafts from the exit head checked after every layer")
    sh = model.shape
    L = sh.n_layers
    tokens = np.asarray(tokens, dtype=np.int64)
    B = len(tokens)
    gamma = np.broadcast_to(np.asarray(0.75 if gamma is None else gamma, dtype=np.float64),
                            (L - 1,))
    forced = np.zeros(B, dtype=np.int64) if forced is None else np.asarray(forced, np.int64)
    pos = cache.lens[:B].copy()
    if np.any(pos >= cache.max_seq):
        raise ValueError("cache full")
    h = model.tok_emb[tokens].copy()
    exited = np.zeros(B, dtype=bool)
    e = np.full(B, L, dtype=np.int32)
    p_rec = np.full((B, L - 1), np.nan)
    head_max = np.full((B, L - 1), np.nan)
    hidden = [h.copy()] if trace else None
    exit_logits = {}   # sampled decoding: the exit head's logits of each row at its exit layer
    for l in range(1, L + 1):
        bb = np.nonzero(~exited)[0]
        ex = np.nonzero(exited)[0]
        decide = heads and l < L and len(bb) > 0 and l % check_every == 0
        h_in = h[bb].copy() if decide and criterion == "sts" else None
        if len(bb):
            _layer_rows(model, cache, l, bb, h, pos, use_exit=False)
        if len(ex):
            _layer_rows(model, cache, l, ex, h, pos, use_exit=True)
        if decide:
            hl = None
            if criterion == "head":
                p, hl = exit_head(model, l, h[bb])
                head_max[bb, l - 1] = np.abs(hl).max(axis=-1)
            else:
                p = state_transition_similarity(h_in, h[bb])
            p_rec[bb, l - 1] = p
            free = [i for i, b in enumerate(bb) if forced[b] == 0]
            batch_go = bool(free) and min(p[i] for i in free) > gamma[l - 1]
            for i, b in enumerate(bb):
                if forced[b] > 0:
                    go = l == forced[b]
                elif exit_rule == "batch_min":
                    go = batch_go
                else:
                    go = p[i] > gamma[l - 1]
                if go:
                    exited[b] = True
                    e[b] = l
                    if sampled:
                        exit_logits[b] = hl[i]
        elif heads and l < L:   # not a check layer: only forced exits
            for b in bb:
                if forced[b] == l:
                    exited[b] = True
                    e[b] = l
        if trace:
            hidden.append(h.copy())
    tok, gap, logits = final_head(model, h)
    info = {"p": p_rec, "head_absmax": head_max, "gap": gap, "logits": logits}
    if sampled:
        info["sample"] = []
        for b in range(B):
            t, si = sample_token(logits[b], exit_logits.get(b), temperature, seed, int(pos[b]), b)
            tok[b] = t
            info["sample"].append(si)
    cache.lens[:B] += 1
    if trace:
        info["hidden"] = np.stack(hidden, axis=1)
    return tok, e, info


def prefill(model: OracleModel, cache: KVCache, prompts, trace: bool = False, exit_tau=None):
    """Backbone pass over every prompt position of sequences 0..B-1.

    Layer-major: each layer runs on all positions, with causal attention over
    the cached keys.  Returns ``(first_tokens [B], info)`` with ``gap`` and
    ``logits`` of the last position, ``exit`` [B] (each sequence's exit
    layer; L without exits) and ``hidden`` [B, P, L+1, d] with trace.

    ``exit_tau`` (thresholds tau_1..tau_{L-1}, scalar broadcasts): River-LLM's
    sequence-level exit in the prefill (River-LLM explainer, section 6.1: in
    the prefill all tokens leave at the same layer; section 5.2: the exit fires
    when the minimum state transition similarity over the tokens exceeds tau).
    Reading: per sequence, over its prompt's tokens; after layer l < L a
    sequence still on the backbone exits iff the smallest similarity of its
    tokens is > tau_l, and its later layers run on the exit copies for every
    one of its tokens.  None: full depth for every sequence.
    """
    sh = model.shape
    L, H, Hkv, hd = sh.n_layers, sh.n_heads, sh.n_kv_heads, sh.head_dim
    prompts = np.asarray(prompts, dtype=np.int64)
    B, P = prompts.shape
    pos0 = cache.lens[:B].copy()
    if np.any(pos0 + P > cache.max_seq):
        raise ValueError("cache full")
    tau = None
    if exit_tau is not None:
        tau = np.broadcast_to(np.asarray(exit_tau, dtype=np.float64), (max(L - 1, 0),))
    cos, sin = model.rope(int(pos0.max()) + P)
    h = model.tok_emb[prompts].copy()                 # [B, P, d]
    hidden = [h.copy()] if trace else None
    exited = np.zeros(B, dtype=bool)
    e = np.full(B, L, dtype=np.int32)
    group = H // Hkv
    scale = 1.0 / np.sqrt(hd)
    for l in range(1, L + 1):
        h_in = h.copy() if tau is not None else None
        for use_exit in (False, True):
            rows = np.nonzero(exited == use_exit)[0]
            if len(rows) == 0:
                continue
            W = model.w_exit if use_exit else model.w
            hr = h[rows]
            n = len(rows)
            x = rmsnorm(hr, model.w(l, "attn_norm"), sh.rms_eps)
            q = bf16_round(lin(x, W(l, "wq"))).reshape(n, P, H, hd)
            k = bf16_round(lin(x, W(l, "wk"))).reshape(n, P, Hkv, hd)
            v = bf16_round(lin(x, W(l, "wv"))).reshape(n, P, Hkv, hd)
            o = np.empty((n, P, H, hd))
            for i, b in enumerate(rows):
                ap = pos0[b] + np.arange(P)
                c, s_ = cos[ap][:, None, :], sin[ap][:, None, :]
                qr = apply_rope(q[i], c, s_)
                kr = apply_rope(k[i], c, s_)
                for t in range(P):
                    cache.store(l, b, int(ap[t]), kr[t], v[i, t])
                nk = int(pos0[b]) + P
                Kb, Vb = cache.keys(l, b, nk)
                for hh in range(H):
                    j = hh // group
                    sc = (qr[:, hh] @ Kb[j].T) * scale           # [P, nk]
                    mask = np.arange(nk)[None, :] > ap[:, None]  # causal
                    sc = np.where(mask, -np.inf, sc)
                    pi = np.exp(sc - sc.max(axis=1, keepdims=True))
                    pi /= pi.sum(axis=1, keepdims=True)
                    o[i, :, hh] = pi @ Vb[j]
            o = bf16_round(o.reshape(n, P, H * hd))
            hr = hr + lin(o, W(l, "wo"))
            x = rmsnorm(hr, model.w(l, "ffn_norm"), sh.rms_eps)
            a = bf16_round(silu(lin(x, W(l, "w_gate"))) * lin(x, W(l, "w_up")))
            h[rows] = hr + lin(a, W(l, "w_down"))
        if tau is not None and l < L:
            for b in np.nonzero(~exited)[0]:
                if state_transition_similarity(h_in[b], h[b]).min() > tau[l - 1]:
                    exited[b] = True
                    e[b] = l
        if trace:
            hidden.append(h.copy())
    tok, gap, logits = final_head(model, h[:, -1])
    cache.lens[:B] += P
    info = {"gap": gap, "logits": logits, "h_last": h[:, -1].copy(), "exit": e}
    if trace:
        info["hidden"] = np.stack(hidden, axis=2)
    return tok, info


def generate(model: OracleModel, cache: KVCache, prompts, steps: int, gamma=None,
             forced_fn=None, criterion: str = "head", check_every: int = 1, exit_rule: str = "sequence",
             temperature: float = 0.0, seed: int = 0):
    """Prefill, then ``steps`` decode steps feeding back each greedy token.

    ``forced_fn(step)`` may return a forced-exit array for a step.  Returns
    ``(tokens [B, steps+1], exits [B, steps])``.
    """
    tok, _ = prefill(model, cache, prompts)
    toks, exits = [tok], []
    for s in range(steps):
        f = forced_fn(s) if forced_fn is not None else None
        tok, e, _ = decode_step(model, cache, tok, gamma=gamma, forced=f, criterion=criterion,
                                check_every=check_every, exit_rule=exit_rule, temperature=temperature, seed=seed)
        toks.append(tok)
        exits.append(e)
    return np.stack(toks, axis=1), (np.stack(exits, axis=1) if exits else
                                     np.zeros((len(tok), 0), np.int32))
