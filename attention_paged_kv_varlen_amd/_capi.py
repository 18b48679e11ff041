"""ctypes binding of libpagedattn: the C entry points under the same names.

Argument marshalling only: every step of the attention runs in the HIP
library.  Tensors are passed by ``data_ptr()``; torch is used for device
memory and streams.  Loading fails loudly when ``libpagedattn.so`` has not
been built (``python -m attention_paged_kv_varlen_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP, PA_ERR_OOM = range(5)
PA_BF16, PA_FP32 = 0, 1
PA_KV_SAME, PA_KV_FP8_E4M3 = 0, 1
PA_KV_NHD, PA_KV_HND = 0, 1
(PA_ARRAY_ORDER, PA_ARRAY_IS_DECODE, PA_ARRAY_PREFIX_BLOCKS, PA_ARRAY_ROW_PARTIALS, PA_ARRAY_DECODE_LISTS,
 PA_ARRAY_DECODE_SPANS) = range(6)

# Every symbol include/pagedattn.h declares.
EXPORTED = (
    "pa_kv_cache_shape", "pa_kv_cache_stride_order", "pa_plan_create", "pa_plan_get_info", "pa_plan_get_array",
    "pa_plan_workspace_bytes", "pa_plan_check_metadata", "pa_forward", "pa_forward_noalloc", "pa_forward_fp8", "pa_merge_states", "pa_gather_kv", "pa_write_kv",
    "pa_write_kv_fp8", "pa_plan_destroy", "pa_status_string", "pa_last_error", "pa_profile_start",
    "pa_profile_stop",
)


class pa_params(ctypes.Structure):
    _fields_ = [
        ("num_seqs", c_int32), ("num_heads", c_int32), ("num_kv_heads", c_int32),
        ("head_size", c_int32), ("block_size", c_int32), ("num_blocks", c_int32),
        ("max_blocks_per_seq", c_int32), ("dtype", c_int32), ("causal", c_int32),
        ("common_prefix_len", c_int32), ("kv_split_tokens", c_int32), ("scale", c_float),
        ("kv_dtype", c_int32), ("kv_layout", c_int32), ("check_metadata", c_int32),
    ]


class pa_plan_info(ctypes.Structure):
    _fields_ = [
        ("num_seqs", c_int32), ("num_tokens", c_int32), ("num_decodes", c_int32),
        ("num_decode_tokens", c_int32), ("num_prefills", c_int32), ("num_prefill_tokens", c_int32),
        ("common_prefix_len", c_int32), ("num_prefix_blocks", c_int32),
        ("num_decode_items", c_int32), ("num_prefill_items", c_int32), ("num_prefix_items", c_int32),
        ("num_merge_rows", c_int32), ("num_partials", c_int32), ("kv_split_tokens", c_int32),
        ("prefill_rows_per_item", c_int32), ("prefill_head_groups", c_int32),
        ("num_decode_lists", c_int32), ("decode_list_tokens", c_int32),
        ("kv_tokens_read", c_int64), ("prefix_tokens_read", c_int64),
        ("decode_tokens_read", c_int64), ("prefill_tokens_read", c_int64),
        ("prefix_tokens_unique", c_int64), ("prefix_beside_decode", c_int32), ("decode_item_keys", c_int32),
        ("decode_list_xcd_budgets", c_int32),
    ]


class pa_kernel_time(ctypes.Structure):
    _fields_ = [("name", c_char * 48), ("launches", c_int32), ("total_ms", c_double), ("min_ms", c_double),
                ("median_ms", c_double), ("max_ms", c_double)]


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded library (loaded once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m attention_paged_kv_varlen_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.pa_kv_cache_shape.argtypes = [c_int64, c_int32, c_int32, c_int32, POINTER(c_int64)]
    L.pa_kv_cache_stride_order.argtypes = [c_int32, POINTER(c_int32)]
    L.pa_plan_create.argtypes = [POINTER(pa_params), POINTER(c_int32), POINTER(c_int32), POINTER(c_int32),
                                 c_int, POINTER(c_void_p)]
    L.pa_plan_get_info.argtypes = [c_void_p, POINTER(pa_plan_info)]
    L.pa_plan_get_array.argtypes = [c_void_p, c_int32, POINTER(c_int32), c_int64, POINTER(c_int64)]
    L.pa_plan_workspace_bytes.argtypes = [c_void_p]
    L.pa_plan_workspace_bytes.restype = c_size_t
    L.pa_plan_check_metadata.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    L.pa_forward.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_size_t, c_void_p]
    L.pa_merge_states.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                  c_int32, c_int32, c_void_p]
    L.pa_gather_kv.argtypes = [c_void_p, c_void_p, c_int32, POINTER(pa_params), c_void_p, c_void_p, c_void_p]
    L.pa_write_kv.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, POINTER(pa_params), c_void_p, c_void_p]
    L.pa_forward_noalloc.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p]
    L.pa_forward_fp8.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    L.pa_write_kv_fp8.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, POINTER(pa_params), c_void_p, c_void_p,
                                  c_int32, c_void_p, c_void_p]
    L.pa_plan_destroy.argtypes = [c_void_p]
    L.pa_plan_destroy.restype = None
    L.pa_status_string.argtypes = [c_int]
    L.pa_status_string.restype = c_char_p
    L.pa_last_error.argtypes = []
    L.pa_last_error.restype = c_char_p
    L.pa_profile_start.argtypes = [c_int32]
    L.pa_profile_stop.argtypes = [POINTER(pa_kernel_time), c_int32, POINTER(c_int32)]
    for name in EXPORTED:
        if name not in ("pa_plan_workspace_bytes", "pa_plan_destroy", "pa_status_string", "pa_last_error"):
            getattr(L, name).restype = c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status != PA_OK:
        L = lib()
        msg = L.pa_last_error().decode() or L.pa_status_string(status).decode()
        raise PagedAttnError(status, msg)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _ptr(x) -> int | None:
    """Device/host address of a tensor (or an int address, or None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owns a pa_plan handle; destroyed with the object."""

    def __init__(self, handle: int, params: pa_params):
        self.handle = handle
        self.params = params

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.pa_plan_destroy(self.handle)
            self.handle = None

    @property
    def _as_parameter_(self):
        return self.handle


def make_params(*, num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks, max_blocks_per_seq,
                dtype, scale, causal=True, common_prefix_len=0, kv_split_tokens=0, kv_dtype="same",
                kv_layout="NHD", check_metadata=False) -> pa_params:
    dt = {"bf16": PA_BF16, "fp32": PA_FP32}.get(dtype, dtype)
    kvt = {"same": PA_KV_SAME, None: PA_KV_SAME, "fp8_e4m3": PA_KV_FP8_E4M3}.get(kv_dtype, kv_dtype)
    lay = {"NHD": PA_KV_NHD, "HND": PA_KV_HND}.get(kv_layout, kv_layout)
    return pa_params(int(num_seqs), int(num_heads), int(num_kv_heads), int(head_size), int(block_size),
                     int(num_blocks), int(max_blocks_per_seq), int(dt), int(bool(causal)),
                     int(common_prefix_len), int(kv_split_tokens), float(scale), int(kvt), int(lay),
                     int(bool(check_metadata)))


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def pa_kv_cache_shape(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int) -> tuple:
    out = (c_int64 * 5)()
    _check(lib().pa_kv_cache_shape(num_blocks, block_size, num_kv_heads, head_size, out))
    return tuple(int(x) for x in out)


def pa_kv_cache_stride_order(layout) -> tuple:
    lay = {"NHD": PA_KV_NHD, "HND": PA_KV_HND}.get(layout, layout)
    out = (c_int32 * 5)()
    _check(lib().pa_kv_cache_stride_order(int(lay), out))
    return tuple(int(x) for x in out)


def pa_plan_create(params: pa_params, query_start_loc, seq_lens, block_table=None, device: int = 0) -> Plan:
    qsl = _i32(query_start_loc)
    sl = _i32(seq_lens)
    bt = None if block_table is None else _i32(block_table)
    if qsl.shape[0] != params.num_seqs + 1 or sl.shape[0] != params.num_seqs:
        raise PagedAttnError(PA_ERR_INVALID_ARG, "query_start_loc / seq_lens length does not match num_seqs")
    if bt is not None and bt.size != params.num_seqs * params.max_blocks_per_seq:
        raise PagedAttnError(PA_ERR_INVALID_ARG, "block_table size does not match num_seqs * max_blocks_per_seq")
    h = c_void_p()
    _check(lib().pa_plan_create(ctypes.byref(params), qsl.ctypes.data_as(POINTER(c_int32)),
                                sl.ctypes.data_as(POINTER(c_int32)),
                                None if bt is None else bt.ctypes.data_as(POINTER(c_int32)), device,
                                ctypes.byref(h)))
    return Plan(h.value, params)


def pa_plan_get_info(plan: Plan) -> dict:
    info = pa_plan_info()
    _check(lib().pa_plan_get_info(plan.handle, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in pa_plan_info._fields_}


def pa_plan_get_array(plan: Plan, which: int) -> np.ndarray:
    n = c_int64(-1)
    st = lib().pa_plan_get_array(plan.handle, which, None, 0, ctypes.byref(n))
    if n.value < 0:  # the length was not reported: unknown array or bad plan
        _check(st)
    out = np.zeros(max(n.value, 0), dtype=np.int32)
    _check(lib().pa_plan_get_array(plan.handle, which, out.ctypes.data_as(POINTER(c_int32)), out.size,
                                   ctypes.byref(n)))
    return out


def pa_plan_workspace_bytes(plan: Plan) -> int:
    return int(lib().pa_plan_workspace_bytes(plan.handle))


def pa_plan_check_metadata(plan: Plan, block_table, query_start_loc=None, seq_lens=None, stream=None) -> None:
    _check(lib().pa_plan_check_metadata(plan.handle, _ptr(block_table), _ptr(query_start_loc), _ptr(seq_lens),
                                        _stream(stream)))


def pa_forward(plan: Plan, q, kv_cache, block_table, query_start_loc, seq_lens, out, lse=None, workspace=None,
               workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_forward(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(query_start_loc),
                            _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(workspace), workspace_bytes,
                            _stream(stream)))


def pa_forward_noalloc(plan: Plan, q, kv_cache, block_table, query_start_loc, seq_lens, out, lse=None,
                       stream=None) -> None:
    _check(lib().pa_forward_noalloc(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(query_start_loc),
                                    _ptr(seq_lens), _ptr(out), _ptr(lse), _stream(stream)))


def pa_forward_fp8(plan: Plan, q, kv_cache, block_table, query_start_loc, seq_lens, k_scale, v_scale, out, lse=None,
                   workspace=None, workspace_bytes=None, num_scales=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if num_scales is None:
        num_scales = int(k_scale.numel())
    _check(lib().pa_forward_fp8(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(query_start_loc),
                                _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale), int(num_scales), _ptr(out), _ptr(lse),
                                _ptr(workspace), workspace_bytes, _stream(stream)))


def pa_merge_states(o_a, lse_a, o_b, lse_b, o_out, lse_out=None, *, num_tokens=None, num_heads=None,
                    head_size=None, dtype=None, stream=None) -> None:
    if num_tokens is None:
        num_tokens, num_heads, head_size = (int(s) for s in o_a.shape)
    if dtype is None:
        import torch
        dtype = PA_BF16 if o_a.dtype == torch.bfloat16 else PA_FP32
    _check(lib().pa_merge_states(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o_out), _ptr(lse_out),
                                 num_tokens, num_heads, head_size, dtype, _stream(stream)))


def pa_gather_kv(kv_cache, block_table_row, seq_len: int, params: pa_params, k_out, v_out, stream=None) -> None:
    _check(lib().pa_gather_kv(_ptr(kv_cache), _ptr(block_table_row), int(seq_len), ctypes.byref(params),
                              _ptr(k_out), _ptr(v_out), _stream(stream)))


def pa_write_kv(key, value, slot_mapping, num_tokens: int, params: pa_params, kv_cache, stream=None) -> None:
    _check(lib().pa_write_kv(_ptr(key), _ptr(value), _ptr(slot_mapping), int(num_tokens), ctypes.byref(params),
                             _ptr(kv_cache), _stream(stream)))


def pa_write_kv_fp8(key, value, slot_mapping, num_tokens: int, params: pa_params, k_scale, v_scale, kv_cache,
                    num_scales=None, stream=None) -> None:
    if num_scales is None:
        num_scales = int(k_scale.numel())
    _check(lib().pa_write_kv_fp8(_ptr(key), _ptr(value), _ptr(slot_mapping), int(num_tokens), ctypes.byref(params),
                                 _ptr(k_scale), _ptr(v_scale), int(num_scales), _ptr(kv_cache), _stream(stream)))


def pa_plan_destroy(plan: Plan) -> None:
    if plan.handle:
        lib().pa_plan_destroy(plan.handle)
        plan.handle = None


def pa_status_string(status: int) -> str:
    return lib().pa_status_string(status).decode()


def pa_last_error() -> str:
    return lib().pa_last_error().decode()


def pa_profile_start(max_launches: int) -> None:
    _check(lib().pa_profile_start(max_launches))


def pa_profile_stop(capacity: int = 64) -> list:
    buf = (pa_kernel_time * capacity)()
    n = c_int32()
    _check(lib().pa_profile_stop(buf, capacity, ctypes.byref(n)))
    return [{"name": buf[i].name.decode(), "launches": buf[i].launches, "total_ms": buf[i].total_ms,
             "min_ms": buf[i].min_ms, "median_ms": buf[i].median_ms, "max_ms": buf[i].max_ms}
            for i in range(n.value)]
