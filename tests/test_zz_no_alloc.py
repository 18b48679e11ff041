"""pa_forward_noalloc: pa_forward with its workspace in the library's static
device array.  Its output must equal pa_forward's (same kernels) bit for bit,
on two calls in a row, the second with a smaller batch (the array keeps the
first call's contents), and it must refuse a plan whose workspace exceeds the
array, launching nothing; captured into a HIP graph (a caller that cannot
allocate), every replay must give the eager result."""
import numpy as np
import pytest

import attention_paged_kv_varlen_amd as pa
from tests.gpu_helpers import announce, assert_close, oracle_full
from workloads import make_batch

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def _device(batch, split):
    return pa.to_device(batch.q, batch.kv_cache, batch.block_table, batch.query_start_loc, batch.seq_lens,
                        num_heads=batch.num_heads, num_kv_heads=batch.num_kv_heads, head_size=batch.head_size,
                        block_size=batch.block_size, dtype=batch.dtype, scale=batch.scale, kv_split_tokens=split,
                        common_prefix_len=batch.common_prefix_len)


def test_noalloc_matches_forward_on_two_calls():
    import torch
    big = make_batch([1] * 12 + [70, 33], [3000, 17, 900, 4096, 2500, 64, 1, 333, 1200, 2048, 700, 1500, 300, 33],
                     num_heads=16, num_kv_heads=2, head_size=128, block_size=16, seed=80)
    small = make_batch([1, 1, 20], [500, 40, 120], num_heads=8, num_kv_heads=2, head_size=128, block_size=32, seed=81)
    for name, batch, split in (("large", big, 96), ("smaller", small, 64)):
        announce(f"noalloc {name}: B={batch.num_seqs} T={batch.num_tokens}")
        db = _device(batch, split)
        need = pa.pa_plan_workspace_bytes(db.plan)
        assert 0 < need <= SCRATCH_BYTES
        db.forward()
        torch.cuda.synchronize()
        want_o, want_l = db.out.clone(), db.lse.clone()
        db.out.fill_(7.0)
        db.lse.fill_(7.0)
        pa.pa_forward_noalloc(db.plan, db.q, db.kv_cache, db.block_table, db.query_start_loc, db.seq_lens, db.out,
                              db.lse)
        torch.cuda.synchronize()
        assert torch.equal(db.out, want_o) and torch.equal(db.lse, want_l), name
        ref_o, ref_l = oracle_full(batch)
        assert_close(db.out.float().cpu().numpy().astype(np.float64), db.lse.cpu().numpy().astype(np.float64),
                     ref_o, ref_l, f"noalloc {name} vs oracle")


def test_noalloc_rejects_a_plan_larger_than_the_scratch():
    import torch
    announce("noalloc: workspace beyond the static array")
    # 5 decodes of 16384 keys cut into 32-key parts: 2560 partial records of
    # 64 heads x (128 + 1) floats, about 85 MB
    lens = [16384] * 5
    params = pa.make_params(num_seqs=5, num_heads=64, num_kv_heads=8, head_size=128, block_size=16, num_blocks=5 * 1024,
                            max_blocks_per_seq=1024, dtype="bf16", scale=0.1, kv_split_tokens=32)
    plan = pa.pa_plan_create(params, np.arange(6), lens, None, device=0)
    assert pa.pa_plan_workspace_bytes(plan) > SCRATCH_BYTES
    out = torch.full((5, 64, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pa.PagedAttnError) as ei:
        pa.pa_forward_noalloc(plan, 16, 16, 16, None, None, out, None)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool(torch.all(out.float() == 3.0))


def test_noalloc_in_a_graph():
    import torch
    batch = make_batch([1, 1, 1, 30], [700, 64, 1500, 130], num_heads=8, num_kv_heads=2, head_size=128,
                       block_size=16, seed=82)
    announce("noalloc captured into a graph")
    db = _device(batch, 64)
    assert pa.pa_plan_workspace_bytes(db.plan) > 0
    db.forward()
    torch.cuda.synchronize()
    want_o, want_l = db.out.clone(), db.lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the capture stream (the first call looks the array up)
        pa.pa_forward_noalloc(db.plan, db.q, db.kv_cache, db.block_table, db.query_start_loc, db.seq_lens, db.out,
                              db.lse, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.pa_forward_noalloc(db.plan, db.q, db.kv_cache, db.block_table, db.query_start_loc, db.seq_lens, db.out,
                              db.lse)
    for rep in range(3):
        db.out.zero_()
        db.lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(db.out, want_o) and torch.equal(db.lse, want_l), f"replay {rep} differs"
        db.forward()  # eager work between replays
        torch.cuda.synchronize()
