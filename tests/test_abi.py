"""The C-ABI library loads on a machine without a GPU and exports every symbol
that include/pagedattn.h declares; host-only calls work without a device."""
import os
import re
import subprocess

import pytest

import attention_paged_kv_varlen_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(pa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = pa.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (pa_[a-z_]+)\b", nm))
    assert set(declared_functions()) <= exported


def test_kv_cache_shape_matches_the_page():
    # «FlashAttention y FlashInfer», §Flujo de datos: (num_blocks, 2, block_size, num_kv_heads, head_size)
    assert pa.pa_kv_cache_shape(76700, 16, 8, 128) == (76700, 2, 16, 8, 128)
    for bs in (8, 24, 0):
        with pytest.raises(pa.PagedAttnError) as ei:
            pa.pa_kv_cache_shape(10, bs, 8, 128)
        assert ei.value.status == pa.PA_ERR_INVALID_ARG


def test_status_strings_and_last_error():
    assert pa.pa_status_string(pa.PA_OK) == "ok"
    assert pa.pa_status_string(pa.PA_ERR_UNSUPPORTED) == "unsupported"
    with pytest.raises(pa.PagedAttnError):
        pa.pa_kv_cache_shape(10, 24, 8, 128)
    assert "multiple of 16" in pa.pa_last_error()


def test_profile_stop_without_session_is_an_error():
    with pytest.raises(pa.PagedAttnError):
        pa.pa_profile_stop()
