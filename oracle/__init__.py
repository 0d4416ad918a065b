"""CPU oracle for the KV-shared early-exit decode step (test infrastructure).

This package is test infrastructure, not product code.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or run anything in it.  It shares no code with the HIP path
(``kv_shared_exit_amd``); the only common dependency is the seeded input
generator ``synth``, which holds no arithmetic of the method.

Sources (page titles and sections of the surveyed web pages):
  * "River-LLM 深度解析" (River-LLM explainer): section 3.1 (attention formula and
    KV cache), section 4.1-4.3 (exit layers as 4-bit copies that share the KV
    store), section 8.1 (symmetric int4 quantiser: scale = max|w| / 7, codes
    clamped to [-8, 7]), section 8.2 (shared KV cache), section 6.1 (two-phase
    generation: prefill, then per-token decode steps).
  * CALM explainer ("Confident Adaptive Language Modeling"): section 2.1
    (confidence from a peaked softmax), section 2.2 (decisions per token and per
    layer), section 3.1 (the layer loop with a per-layer threshold).
  * "大语言模型解码加速：自适应层并行机制解析" (AdaDecode explainer): section 2.1
    (intermediate head h^(l) T^(l) E^T), section 2.2 (exit when the top-1
    probability exceeds gamma, default 0.75).

Arithmetic is float64 throughout.  Values are rounded to bf16 exactly where the
decode step stores them as 16-bit data (weights, GEMV inputs, K/V cache
entries, attention output, SwiGLU output, exit-head projection); the residual
stream, logits and softmax stay in float64.

Parity status of each function is recorded in its docstring; every function
here is pinned by a ``-m "not gpu"`` test except where it says otherwise.
"""
from .numerics import bf16_round
from .quant import quantize_int4, dequantize_int4
from .model import OracleModel, KVCache, decode_step, prefill, generate

__all__ = ["bf16_round", "quantize_int4", "dequantize_int4", "OracleModel", "KVCache",
           "decode_step", "prefill", "generate"]
