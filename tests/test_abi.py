"""The C ABI library loads and exports every symbol include/ee.h declares (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ee.h")
LIB = os.path.join(ROOT, "kv_shared_exit_amd", "libee.so")


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:ee_status|const char \*)\s*(ee_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    names = declared()
    for n in ("ee_create_model", "ee_prefill", "ee_decode_step", "ee_kv_cache_create",
              "ee_kv_cache_read", "ee_kv_cache_destroy", "ee_last_error"):
        assert n in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="libee.so not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for n in declared():
        assert hasattr(lib, n), n
    from kv_shared_exit_amd import _binding
    assert sorted(_binding.EXPORTS) == declared()


@pytest.mark.skipif(not os.path.exists(LIB), reason="libee.so not built")
def test_null_arguments_are_rejected_without_a_gpu():
    from kv_shared_exit_amd import _binding as B
    lib = B.load()
    h = ctypes.c_void_p()
    assert lib.ee_create_model(None, None, None, ctypes.byref(h)) == B.EE_ERR_INVALID_ARG
    assert b"null" in lib.ee_last_error()
    assert lib.ee_destroy_model(None) == B.EE_OK
    assert lib.ee_kv_cache_destroy(None) == B.EE_OK
