"""ctypes binding of libee (include/ee.h): argument marshalling only.

Every computation of the decode step runs in libee's HIP kernels; this module
only converts Python and torch objects to the C ABI's plain pointers and sizes
and raises ``EEError`` on a non-zero status.  Importing it never falls back to
anything: if libee.so is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libee.so")

EE_OK = 0
EE_ERR_INVALID_ARG = -1
EE_ERR_OUT_OF_MEMORY = -2
EE_ERR_HIP = -3
EE_ERR_CACHE_FULL = -4
EE_ERR_SHAPE = -5
EE_ERR_NOT_WRITTEN = -6
EE_ERR_UNSUPPORTED = -7
EE_EXIT_INT4 = 0
EE_EXIT_BF16 = 1
EE_EXIT_NONE = 2
EE_CRIT_HEAD = 0
EE_CRIT_STS = 1
EE_RULE_SEQUENCE = 0
EE_RULE_BATCH_MIN = 1
EE_KV_TRACK_OCCUPANCY = 1

EXPORTS = [
    "ee_create_model", "ee_destroy_model", "ee_kv_cache_bytes", "ee_kv_cache_create",
    "ee_kv_cache_reset", "ee_kv_cache_rollback", "ee_kv_cache_lengths", "ee_kv_cache_read", "ee_kv_cache_occupancy",
    "ee_kv_cache_destroy", "ee_prefill", "ee_decode_step", "ee_decode_step_static", "ee_exit_weights_read",
    "ee_profile_enable", "ee_profile_read", "ee_last_error",
]


class EEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libee status {status}: {msg}")
        self.status = status


class ModelConfig(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ff", C.c_int32),
                ("vocab", C.c_int32), ("group_size", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_float), ("exit_mode", C.c_int32), ("max_batch", C.c_int32),
                ("max_positions", C.c_int32), ("criterion", C.c_int32), ("check_every", C.c_int32),
                ("exit_rule", C.c_int32), ("temperature", C.c_float), ("sample_seed", C.c_uint32),
                ("prefill_exit", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm",
                                          "w_gate", "w_up", "w_down", "head_T")]


class Weights(C.Structure):
    _fields_ = [("tok_emb", C.c_void_p), ("lm_head", C.c_void_p), ("final_norm", C.c_void_p),
                ("layers", C.POINTER(LayerWeights))]


class StepDebug(C.Structure):
    _fields_ = [("p_top1", C.c_void_p), ("logits", C.c_void_p), ("hidden", C.c_void_p),
                ("gap", C.c_void_p)]


_lib = None


def load() -> C.CDLL:
    """Load libee.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not found: build it with kv_shared_exit_amd.build.build()")
    lib = C.CDLL(LIB_PATH)
    P, I32, U32, SZ = C.c_void_p, C.c_int32, C.c_uint32, C.c_size_t
    sig = {
        "ee_create_model": [C.POINTER(ModelConfig), C.POINTER(Weights), P, C.POINTER(P)],
        "ee_destroy_model": [P],
        "ee_kv_cache_bytes": [P, I32, I32, C.POINTER(SZ)],
        "ee_kv_cache_create": [P, I32, I32, P, SZ, U32, C.POINTER(P)],
        "ee_kv_cache_reset": [P, I32],
        "ee_kv_cache_rollback": [P, I32, I32],
        "ee_kv_cache_lengths": [P, P],
        "ee_kv_cache_read": [P, I32, I32, I32, I32, P, P],
        "ee_kv_cache_occupancy": [P, P],
        "ee_kv_cache_destroy": [P],
        "ee_prefill": [P, P, I32, P, I32, P, P, P, P],
        "ee_decode_step": [P, P, I32, P, P, P, P, P, P, P],
        "ee_decode_step_static": [P, P, I32, P, P, P, P, P, P],
        "ee_exit_weights_read": [P, I32, I32, I32, I32, P, P],
        "ee_profile_enable": [P, I32],
        "ee_profile_read": [P, I32, C.POINTER(C.c_int64), C.POINTER(C.c_double)],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = C.c_int32
    lib.ee_last_error.argtypes = []
    lib.ee_last_error.restype = C.c_char_p
    _lib = lib
    return lib


def check(status: int):
    if status != EE_OK:
        raise EEError(status, load().ee_last_error().decode())


def _ptr(a):
    """Host pointer of a contiguous numpy array (None passes NULL)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)
