"""Edge cases on the GPU, through the C ABI, against the CPU oracle: an empty
batch, the smallest decode and prefill, very long sequences, many sequences,
and wide query-head groups."""
import numpy as np
import pytest

import attention_paged_kv_varlen_amd as pa
import oracle
from tests.gpu_helpers import announce, assert_close, oracle_full, run_gpu
from workloads import make_batch

pytestmark = pytest.mark.gpu


def test_empty_batch_launches_nothing():
    import torch
    announce("empty batch")
    params = pa.make_params(num_seqs=0, num_heads=8, num_kv_heads=2, head_size=128, block_size=16, num_blocks=4,
                            max_blocks_per_seq=1, dtype="bf16", scale=0.1)
    plan = pa.pa_plan_create(params, [0], [], np.zeros((0, 1), np.int32), device=0)
    assert pa.pa_plan_get_info(plan)["num_tokens"] == 0
    assert pa.pa_plan_workspace_bytes(plan) == 0
    pa.pa_forward(plan, 0, 0, 0, None, None, 0)  # no rows: nothing is launched or read
    torch.cuda.synchronize()


def test_smallest_decodes_and_prefills():
    # one-key decodes, two-token prefills with and without context, a one-token
    # chunk boundary exactly at a page end
    qlens = [1, 1, 2, 2, 1, 2]
    lens = [1, 2, 2, 18, 16, 32]
    b = make_batch(qlens, lens, num_heads=8, num_kv_heads=2, head_size=128, block_size=16, seed=70)
    announce("smallest decodes and prefills")
    out, lse, _ = run_gpu(b)
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, "smallest")


@pytest.mark.parametrize("layout,bs", [("NHD", 16), ("HND", 1024)])
def test_very_long_decode(layout, bs):
    # a 131072-token decode beside short ones (the long one is split into many
    # parts and merged)
    lens = [131072, 5, 4097, 1]
    b = make_batch([1] * 4, lens, num_heads=32, num_kv_heads=8, head_size=128, block_size=bs, seed=71,
                   kv_layout=layout)
    announce(f"very long decode {layout} bs={bs}")
    out, lse, db = run_gpu(b)
    assert pa.pa_plan_get_info(db.plan)["num_merge_rows"] >= 1
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, f"long decode {layout}")


def test_long_chunk_sampled_rows():
    # a 512-token chunk after 32768 tokens of context beside decodes; sampled
    # rows (first, last, a spread in between) against the oracle row by row
    qlens = [1, 1, 512]
    lens = [9000, 300, 32768 + 512]
    b = make_batch(qlens, lens, num_heads=16, num_kv_heads=2, head_size=128, block_size=64, seed=72)
    announce("long chunk")
    out, lse, _ = run_gpu(b)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    rows = np.array([0, 1, 2, 3, 100, 257, 400, 512, 513], dtype=np.int64)
    ro, rl = oracle.attention_rows(b.q, b.kv_cache, b.block_table, b.query_start_loc, b.seq_lens, b.scale, rows)
    assert_close(out[rows], lse[rows], ro, rl, "long chunk rows")


def test_many_short_decodes():
    rng = np.random.default_rng(73)
    lens = rng.integers(1, 65, size=2048).tolist()
    b = make_batch([1] * len(lens), lens, num_heads=8, num_kv_heads=2, head_size=64, block_size=16, seed=74)
    announce("2048 short decodes")
    out, lse, _ = run_gpu(b)
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, "many short decodes")


@pytest.mark.parametrize("heads", [(128, 8), (64, 1)])
def test_wide_groups(heads):
    # g = 16 (one 16-column group) and g = 64 (four groups per KV head)
    b = make_batch([1, 1, 40, 1], [300, 1, 90, 1200], num_heads=heads[0], num_kv_heads=heads[1], head_size=128,
                   block_size=16, seed=75)
    announce(f"wide groups H={heads}")
    out, lse, _ = run_gpu(b)
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, f"groups {heads}")


@pytest.mark.parametrize("kv_dtype,split", [("same", 0), ("same", 32), ("same", 64), ("same", 96),
                                            ("fp8_e4m3", 0), ("fp8_e4m3", 32)])
def test_every_short_decode_length(kv_dtype, split):
    # decodes of every length from 1 to 160 keys: work items that end after
    # one 32-key step, after an even or an odd number of steps, at every
    # offset inside a 16-key page; automatic lists (items cut on 32-key
    # boundaries, several sequences per list) and explicit splits
    lens = list(range(1, 161))
    b = make_batch([1] * len(lens), lens, num_heads=32, num_kv_heads=8, head_size=128, block_size=16, seed=76,
                   kv_dtype=kv_dtype)
    announce(f"every short decode length {kv_dtype} split={split}")
    out, lse, db = run_gpu(b, kv_split_tokens=split)
    info = pa.pa_plan_get_info(db.plan)
    if split == 0:
        assert info["decode_list_tokens"] > 0
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, f"short lengths {kv_dtype} split={split}")


@pytest.mark.parametrize("dtype,head_size", [("bf16", 128), ("fp32", 64)])
@pytest.mark.parametrize("scale", [4.0, 1.0, 1e-3])
def test_extreme_softmax_scales(dtype, head_size, scale):
    # scores of N(0,1) rows times a large scale span hundreds in the exponent:
    # the running max moves by more than the speculative limit and the lazy
    # threshold again and again (rescale paths), and the LSE is large; a tiny
    # scale makes the softmax nearly flat (the mean of V).  With a peaked
    # softmax a bf16 output is nearly one V element, rounded to bf16: half an
    # ulp of a value in [4, 8) is 2^-7, most of the error seen at large scales
    qlens = [1, 1, 1, 40, 150]
    lens = [1, 300, 2100, 337, 150]
    b = make_batch(qlens, lens, num_heads=8, num_kv_heads=2, head_size=head_size, block_size=16, seed=77,
                   dtype=dtype, scale=scale)
    announce(f"extreme scale {scale} {dtype} d={head_size}")
    out, lse, _ = run_gpu(b)
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, f"scale {scale} {dtype}")
