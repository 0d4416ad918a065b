"""KV-shared early-exit decode on MI355X (gfx950): libee (HIP kernels behind a C ABI)
and its Python binding.  The HIP library is required: nothing here falls back to
another implementation."""
from ._binding import EEError, load, EE_EXIT_INT4, EE_EXIT_BF16, EE_EXIT_NONE, EE_CRIT_HEAD, EE_CRIT_STS, EE_RULE_SEQUENCE, EE_RULE_BATCH_MIN  # noqa: F401
from .api import Model, KVCache, upload_weights, prefill, decode_step  # noqa: F401
