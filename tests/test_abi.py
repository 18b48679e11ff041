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
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(pa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = pa.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (pa_[a-z0-9_]+)\b", nm))
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


def test_write_kv_validates_before_any_launch():
    """pa_write_kv checks its arguments on the host: nothing runs on a device."""
    import attention_paged_kv_varlen_amd as pa
    p = pa.make_params(num_seqs=1, num_heads=2, num_kv_heads=2, head_size=128, block_size=16, num_blocks=4,
                       max_blocks_per_seq=4, dtype="bf16", scale=0.1)
    pa.pa_write_kv(None, None, None, 0, p, None, stream=0)  # no tokens: nothing to do
    for args, status in (
        ((16, 16, 16, -1, p), pa.PA_ERR_INVALID_ARG),          # negative count
        ((None, 16, 16, 3, p), pa.PA_ERR_INVALID_ARG),         # NULL key
        ((8, 16, 16, 3, p), pa.PA_ERR_INVALID_ARG),            # key not 16-byte aligned
        ((16, 16, 16, 3, pa.make_params(num_seqs=1, num_heads=2, num_kv_heads=2, head_size=128, block_size=24,
                                        num_blocks=4, max_blocks_per_seq=4, dtype="bf16", scale=0.1)),
         pa.PA_ERR_INVALID_ARG),                               # block size not a multiple of 16
        ((16, 16, 16, 3, pa.make_params(num_seqs=1, num_heads=1, num_kv_heads=1, head_size=4, block_size=16,
                                        num_blocks=4, max_blocks_per_seq=4, dtype="bf16", scale=0.1)),
         pa.PA_ERR_UNSUPPORTED),                               # 8-byte K row
    ):
        key, value, slots, n, params = args
        with pytest.raises(pa.PagedAttnError) as ei:
            pa.pa_write_kv(key, value, slots, n, params, kv_cache=16, stream=0)
        assert ei.value.status == status, args


def _fp8_params(**kw):
    base = dict(num_seqs=2, num_heads=8, num_kv_heads=2, head_size=128, block_size=16, num_blocks=8,
                max_blocks_per_seq=4, dtype="bf16", scale=0.1, kv_dtype="fp8_e4m3")
    base.update(kw)
    return pa.make_params(**base)


def test_e4m3_pool_plan_checks():
    """An e4m3 pool is a plan property: bf16 queries only, a known kv_dtype; the
    prefill tiling follows the head size as for bf16 pools (wide kernel at
    d = 128, general kernel at d = 64)."""
    qsl, sl = [0, 1, 65], [40, 64]
    # group of 8: the wide kernel takes 4 heads x 32 positions per workgroup,
    # the general one 8 heads x 16 positions
    rows = {}
    for d in (128, 64):
        for kvd in ("fp8_e4m3", "same"):
            plan = pa.pa_plan_create(_fp8_params(num_heads=16, head_size=d, kv_dtype=kvd), qsl, sl, device=-1)
            info = pa.pa_plan_get_info(plan)
            assert info["num_decodes"] == 1 and info["num_prefills"] == 1
            rows[d, kvd] = info["prefill_rows_per_item"]
    assert rows == {(128, "fp8_e4m3"): 32, (128, "same"): 32, (64, "fp8_e4m3"): 16, (64, "same"): 16}
    for kw, status in ((dict(dtype="fp32"), pa.PA_ERR_UNSUPPORTED), (dict(kv_dtype=7), pa.PA_ERR_INVALID_ARG)):
        with pytest.raises(pa.PagedAttnError) as ei:
            pa.pa_plan_create(_fp8_params(**kw), qsl, sl, device=-1)
        assert ei.value.status == status, kw


def test_e4m3_write_validates_before_any_launch():
    p = _fp8_params()
    pa.pa_write_kv_fp8(None, None, None, 0, p, None, None, None, num_scales=1, stream=0)
    for args, status in (
        ((16, 16, 16, 3, p, 16, 16, 3), pa.PA_ERR_INVALID_ARG),                  # 3 scales for 2 heads
        ((16, 16, 16, 3, p, None, 16, 1), pa.PA_ERR_INVALID_ARG),                # NULL scale
        ((16, 8, 16, 3, p, 16, 16, 1), pa.PA_ERR_INVALID_ARG),                   # value not 16-byte aligned
        ((16, 16, 16, 3, _fp8_params(kv_dtype="same"), 16, 16, 1), pa.PA_ERR_INVALID_ARG),  # not an e4m3 pool
        ((16, 16, 16, 3, _fp8_params(dtype="fp32"), 16, 16, 1), pa.PA_ERR_UNSUPPORTED),    # fp32 inputs
        ((16, 16, 16, 3, _fp8_params(head_size=8), 16, 16, 1), pa.PA_ERR_UNSUPPORTED),     # 8-element heads
    ):
        key, value, slots, n, params, ks, vs, ns = args
        with pytest.raises(pa.PagedAttnError) as ei:
            pa.pa_write_kv_fp8(key, value, slots, n, params, ks, vs, kv_cache=16, num_scales=ns, stream=0)
        assert ei.value.status == status, args
    # the plain write refuses an e4m3 pool
    with pytest.raises(pa.PagedAttnError) as ei:
        pa.pa_write_kv(16, 16, 16, 3, p, kv_cache=16, stream=0)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG


def test_e4m3_forward_needs_a_device_plan_and_scales():
    plan = pa.pa_plan_create(_fp8_params(), [0, 1, 65], [40, 64], device=-1)
    with pytest.raises(pa.PagedAttnError) as ei:
        pa.pa_forward_fp8(plan, 16, 16, 16, None, None, 16, 16, 16, num_scales=2, stream=0)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG


def test_stride_order_and_layout_checks():
    # «FlashAttention y FlashInfer», §Motivación de diseño: NHD / HND stride orders
    assert pa.pa_kv_cache_stride_order("NHD") == (0, 1, 2, 3, 4)
    assert pa.pa_kv_cache_stride_order("HND") == (0, 1, 3, 2, 4)
    with pytest.raises(pa.PagedAttnError) as ei:
        pa.pa_kv_cache_stride_order(5)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG
    p = pa.make_params(num_seqs=1, num_heads=2, num_kv_heads=2, head_size=128, block_size=1024, num_blocks=4,
                       max_blocks_per_seq=4, dtype="bf16", scale=0.1, kv_layout="HND")
    plan = pa.pa_plan_create(p, [0, 3], [3000], device=-1)   # 1024-token pages plan as any others
    assert pa.pa_plan_get_info(plan)["num_prefills"] == 1
    bad = pa.make_params(num_seqs=1, num_heads=2, num_kv_heads=2, head_size=128, block_size=16, num_blocks=4,
                         max_blocks_per_seq=4, dtype="bf16", scale=0.1, kv_layout=3)
    for call in (lambda: pa.pa_plan_create(bad, [0, 1], [5], device=-1),
                 lambda: pa.pa_write_kv(16, 16, 16, 1, bad, kv_cache=16, stream=0),
                 lambda: pa.pa_gather_kv(16, 16, 1, bad, 16, 16, stream=0)):
        with pytest.raises(pa.PagedAttnError) as ei:
            call()
        assert ei.value.status == pa.PA_ERR_INVALID_ARG


def test_merge_and_gather_reject_misaligned_pointers_before_any_launch():
    # the addresses are never dereferenced: the checks come before any launch
    for o_a, lse_a, dtype in ((4, 16, pa.PA_BF16), (8, 16, pa.PA_FP32), (16, 2, pa.PA_FP32)):
        with pytest.raises(pa.PagedAttnError) as ei:
            pa.pa_merge_states(o_a, lse_a, 16, 16, 16, None, num_tokens=3, num_heads=2, head_size=128,
                               dtype=dtype, stream=0)
        assert ei.value.status == pa.PA_ERR_INVALID_ARG and "aligned" in pa.pa_last_error()
    p = pa.make_params(num_seqs=1, num_heads=2, num_kv_heads=2, head_size=128, block_size=16, num_blocks=4,
                       max_blocks_per_seq=4, dtype="bf16", scale=0.1)
    for kv, bt, k_out in ((8, 16, 16), (16, 2, 16), (16, 16, 24)):
        with pytest.raises(pa.PagedAttnError) as ei:
            pa.pa_gather_kv(kv, bt, 5, p, k_out, 16, stream=0)
        assert ei.value.status == pa.PA_ERR_INVALID_ARG and "aligned" in pa.pa_last_error()
