"""The C ABI's argument checks on the GPU: misaligned pointers, device metadata
that differs from the plan's, and two host threads sharing one plan.  Each
rejected call must leave the outputs untouched (nothing launched)."""
import threading

import numpy as np
import pytest

import attention_paged_kv_varlen_amd as pa
from tests.gpu_helpers import announce, assert_close, oracle_full, run_gpu
from workloads import make_batch

pytestmark = pytest.mark.gpu


def _mixed_batch(seed=70):
    return make_batch([1, 1, 37, 1, 60], [300, 1200, 137, 64, 700], num_heads=8, num_kv_heads=2, head_size=128,
                      block_size=16, seed=seed)


def _device(batch, **kw):
    return pa.to_device(batch.q, batch.kv_cache, batch.block_table, batch.query_start_loc, batch.seq_lens,
                        num_heads=batch.num_heads, num_kv_heads=batch.num_kv_heads, head_size=batch.head_size,
                        block_size=batch.block_size, dtype=batch.dtype, scale=batch.scale, kv_split_tokens=64, **kw)


def _status(fn):
    try:
        fn()
    except pa.PagedAttnError as e:
        return e.status
    return pa.PA_OK


@pytest.mark.parametrize("which", ["q", "out", "kv_cache", "workspace", "lse"])
def test_misaligned_pointer_is_rejected_and_out_untouched(which):
    import torch
    announce(f"misaligned {which}")
    db = _device(_mixed_batch())
    need = pa.pa_plan_workspace_bytes(db.plan)
    assert need > 0
    ws = torch.empty(need + 256, dtype=torch.uint8, device=db.out.device)  # room for an offset pointer
    db.out.fill_(3.0)
    torch.cuda.synchronize()
    args = dict(q=db.q.data_ptr(), kv_cache=db.kv_cache.data_ptr(), out=db.out.data_ptr(), lse=db.lse.data_ptr(),
                workspace=ws.data_ptr())
    # an address inside the same allocation, off the required alignment (16
    # bytes; the LSE needs 4): never dereferenced, the call is rejected first
    args[which] += 2 if which == "lse" else 8
    st = _status(lambda: pa.pa_forward(db.plan, args["q"], args["kv_cache"], db.block_table, db.query_start_loc,
                                       db.seq_lens, args["out"], args["lse"], args["workspace"],
                                       workspace_bytes=need + 128))
    assert st == pa.PA_ERR_INVALID_ARG
    assert "aligned" in pa.pa_last_error()
    torch.cuda.synchronize()
    assert bool(torch.all(db.out.float() == 3.0))


def test_metadata_check_accepts_the_plans_arrays():
    announce("metadata check: consistent")
    db = _device(_mixed_batch())
    pa.pa_plan_check_metadata(db.plan, db.block_table, db.query_start_loc, db.seq_lens)
    pa.pa_plan_check_metadata(db.plan, None, None, None)


@pytest.mark.parametrize("what", ["block_table", "query_start_loc", "seq_lens"])
def test_metadata_check_finds_a_stale_array(what):
    announce(f"metadata check: stale {what}")
    batch = _mixed_batch()
    db = _device(batch)
    bad = {"block_table": db.block_table.clone(), "query_start_loc": db.query_start_loc.clone(),
           "seq_lens": db.seq_lens.clone()}
    if what == "block_table":
        # a used entry of the last sequence now names another (valid) page
        b = batch.num_seqs - 1
        j = (int(batch.seq_lens[b]) - 1) // batch.block_size
        bad[what][b, j] = (int(bad[what][b, j]) + 1) % batch.num_blocks
    elif what == "query_start_loc":
        bad[what][2] += 1
    else:
        bad[what][0] -= 1
    st = _status(lambda: pa.pa_plan_check_metadata(db.plan, bad["block_table"], bad["query_start_loc"],
                                                   bad["seq_lens"]))
    assert st == pa.PA_ERR_INVALID_ARG and "differs" in pa.pa_last_error()


def test_checked_forward_rejects_stale_table_and_runs_on_the_right_one():
    import torch
    announce("forward with check_metadata")
    batch = _mixed_batch()
    db = _device(batch, check_metadata=True)
    stale = db.block_table.clone()
    stale[0, 0] = (int(stale[0, 0]) + 1) % batch.num_blocks
    db.out.fill_(3.0)
    st = _status(lambda: pa.pa_forward(db.plan, db.q, db.kv_cache, stale, db.query_start_loc, db.seq_lens, db.out,
                                       db.lse, db.workspace))
    assert st == pa.PA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert bool(torch.all(db.out.float() == 3.0))
    db.forward()
    torch.cuda.synchronize()
    out = db.out.float().cpu().numpy().astype(np.float64)
    lse = db.lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = oracle_full(batch)
    assert_close(out, lse, ref_o, ref_l, "checked forward")


def test_two_threads_share_one_plan():
    """A plan with decodes and prefills forks onto its side stream; two host
    threads run it concurrently on their own streams, outputs and workspaces.
    Every result must equal the single-thread one bit for bit."""
    import torch
    announce("two threads, one plan")
    batch = _mixed_batch(seed=71)
    ref_o, ref_l, db = run_gpu(batch, kv_split_tokens=64)
    assert pa.pa_plan_get_info(db.plan)["num_prefill_items"] > 0
    want_o = db.out.clone()
    want_l = db.lse.clone()
    n_iter = 20
    outs = [[torch.empty_like(db.out) for _ in range(n_iter)] for _ in range(2)]
    lses = [[torch.empty_like(db.lse) for _ in range(n_iter)] for _ in range(2)]
    wss = [torch.empty_like(db.workspace) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    errors = []

    def worker(k):
        try:
            with torch.cuda.stream(streams[k]):
                for i in range(n_iter):
                    pa.pa_forward(db.plan, db.q, db.kv_cache, db.block_table, db.query_start_loc, db.seq_lens,
                                  outs[k][i], lses[k][i], wss[k], stream=streams[k])
            streams[k].synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        for i in range(n_iter):
            assert torch.equal(outs[k][i], want_o) and torch.equal(lses[k][i], want_l), (k, i)
    ref = oracle_full(batch)
    assert_close(ref_o, ref_l, *ref, "two threads (single-thread result)")
