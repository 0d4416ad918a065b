"""A plain greedy decoder written from torch library calls, used to pin the oracle.

It recomputes the whole sequence with a causal mask at every step (no KV
cache, no incremental state) and uses ``torch.nn.functional.rms_norm``,
``scaled_dot_product_attention(enable_gqa=True)``, ``silu`` and complex
multiplication for the rotary embedding.  bf16 rounding uses round-to-odd into
float32 followed by torch's float32 -> bfloat16 cast, a different algorithm from
the oracle's.  Each layer may be given its own weight dict, so special cases of
the early-exit method (no exit; exit after layer 1 with dequantised layers
2..L) reduce to this decoder with the right per-layer weights.
"""
import numpy as np
import torch
import torch.nn.functional as F


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """float64 -> bf16 value (as float64) in one correct rounding, via round-to-odd float32."""
    f = x.to(torch.float32)
    back = f.to(torch.float64)
    # round toward zero into float32 ...
    away = back.abs() > x.abs()
    f = torch.where(away, torch.nextafter(f, torch.zeros_like(f)), f)
    back = f.to(torch.float64)
    # ... and make it odd when inexact (sticky bit)
    inexact = back != x
    bits = f.view(torch.int32)
    bits = torch.where(inexact, bits | 1, bits)
    return bits.view(torch.float32).to(torch.bfloat16).to(torch.float64)


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float64)


class PlainDecoder:
    def __init__(self, shape, tok_emb, lm_head, final_norm, layers):
        """layers: list of L dicts name -> float64 tensor (attn_norm, wq, ..., w_down)."""
        self.s = shape
        self.tok_emb, self.lm_head, self.final_norm = tok_emb, lm_head, final_norm
        self.layers = layers

    def rot(self, n):
        hd = self.s.head_dim
        inv = self.s.rope_theta ** (-(torch.arange(0, hd, 2, dtype=torch.float64)) / hd)
        ang = torch.arange(n, dtype=torch.float64)[:, None] * inv[None, :]
        c = torch.cos(ang).to(torch.float32).to(torch.float64)
        s = torch.sin(ang).to(torch.float32).to(torch.float64)
        return torch.complex(c, s)

    def rope(self, x, rot):
        # x [T, heads, hd]; pair (i, i + hd/2) is the complex number x_i + j x_{i+hd/2}
        half = x.shape[-1] // 2
        z = torch.complex(x[..., :half], x[..., half:]) * rot[:, None, :]
        return to_bf16(torch.cat([z.real, z.imag], dim=-1))

    def forward(self, tokens):
        """Full causal pass. Returns (hidden [L+1, T, d], logits [T, V], K [L, Hkv, T, hd], V)."""
        s = self.s
        T = len(tokens)
        h = self.tok_emb[torch.as_tensor(tokens, dtype=torch.long)]
        rot = self.rot(T)
        hs, Ks, Vs = [h], [], []
        for lw in self.layers:
            x = to_bf16(F.rms_norm(h, (s.d_model,), weight=lw["attn_norm"], eps=s.rms_eps))
            q = to_bf16(x @ lw["wq"].T).view(T, s.n_heads, s.head_dim)
            k = to_bf16(x @ lw["wk"].T).view(T, s.n_kv_heads, s.head_dim)
            v = to_bf16(x @ lw["wv"].T).view(T, s.n_kv_heads, s.head_dim)
            q, k = self.rope(q, rot), self.rope(k, rot)
            Ks.append(k.transpose(0, 1))
            Vs.append(v.transpose(0, 1))
            o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                               v.transpose(0, 1)[None], is_causal=True,
                                               enable_gqa=True)[0]
            o = to_bf16(o.transpose(0, 1).reshape(T, -1))
            h = h + o @ lw["wo"].T
            x = to_bf16(F.rms_norm(h, (s.d_model,), weight=lw["ffn_norm"], eps=s.rms_eps))
            a = to_bf16(F.silu(x @ lw["w_gate"].T) * (x @ lw["w_up"].T))
            h = h + a @ lw["w_down"].T
            hs.append(h)
        y = to_bf16(F.rms_norm(h, (s.d_model,), weight=self.final_norm, eps=s.rms_eps))
        return torch.stack(hs), y @ self.lm_head.T, torch.stack(Ks), torch.stack(Vs)

    def greedy(self, prompt, steps):
        """Prompt then ``steps`` greedy tokens (lowest index wins ties)."""
        seq = list(prompt)
        out = []
        gaps = []
        for _ in range(steps + 1):
            _, logits, _, _ = self.forward(seq)
            last = logits[-1]
            t = int(torch.argmax(last))
            top = torch.topk(last, 2).values if len(last) > 1 else None
            gaps.append(float(top[0] - top[1]) if top is not None else float("inf"))
            out.append(t)
            seq.append(t)
        return out, gaps
