"""Helpers shared by the GPU tests: run a batch through libpagedattn, compare
with the CPU oracle.  Tolerances: max-abs 2e-2 on outputs, 1e-3 on the
natural-log LSE; gathers and metadata are compared bit for bit."""
from __future__ import annotations

import sys

import numpy as np

OUT_TOL = 2e-2
LSE_TOL = 1e-3


def announce(case: str) -> None:
    """Name the case on stdout before any GPU work starts (flushed)."""
    print(f"\n[gpu-case] {case}", flush=True)
    sys.stdout.flush()


def run_gpu(batch, *, common_prefix_len=None, kv_split_tokens=0, causal=None, q=None, kv_cache=None,
            block_table=None):
    """Plan + forward on cuda:0; returns (out f64, lse f64, DeviceBatch)."""
    import torch

    import attention_paged_kv_varlen_amd as pa
    cp = batch.common_prefix_len if common_prefix_len is None else common_prefix_len
    db = pa.to_device(
        batch.q if q is None else q,
        batch.kv_cache if kv_cache is None else kv_cache,
        batch.block_table if block_table is None else block_table,
        batch.query_start_loc, batch.seq_lens,
        num_heads=batch.num_heads, num_kv_heads=batch.num_kv_heads, head_size=batch.head_size,
        block_size=batch.block_size, dtype=batch.dtype, scale=batch.scale,
        causal=batch.causal if causal is None else causal, common_prefix_len=cp,
        kv_split_tokens=kv_split_tokens, kv_dtype=batch.kv_dtype, k_scale=batch.k_scale, v_scale=batch.v_scale,
        kv_layout=batch.kv_layout)
    db.forward()
    torch.cuda.synchronize()
    out = db.out.float().cpu().numpy().astype(np.float64)
    lse = db.lse.cpu().numpy().astype(np.float64)
    return out, lse, db


def oracle_full(batch, causal=None, q=None, kv_cache=None, block_table=None):
    import oracle
    return oracle.attention(batch.q if q is None else q, batch.kv_cache if kv_cache is None else kv_cache,
                            batch.block_table if block_table is None else block_table,
                            batch.query_start_loc, batch.seq_lens, batch.scale, dtype=batch.dtype,
                            causal=batch.causal if causal is None else causal, kv_dtype=batch.kv_dtype,
                            k_scale=1.0 if batch.k_scale is None else batch.k_scale,
                            v_scale=1.0 if batch.v_scale is None else batch.v_scale, kv_layout=batch.kv_layout)


def assert_close(out, lse, ref_out, ref_lse, what=""):
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    assert np.all(np.isfinite(lse)), f"{what}: non-finite lse"
    eo = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    el = float(np.max(np.abs(lse - ref_lse))) if lse.size else 0.0
    print(f"[gpu-case] {what}: max|out err| {eo:.3e}  max|lse err| {el:.3e}", flush=True)
    assert eo <= OUT_TOL, f"{what}: out error {eo}"
    assert el <= LSE_TOL, f"{what}: lse error {el}"
    return eo, el


def sample_rows(batch, per_seq=4, max_seqs=24, seed=0):
    """A spread of token rows: every decode row of some sequences, and the first,
    last and a few middle rows of prefills; always includes the longest and
    shortest sequence."""
    rng = np.random.default_rng(seed)
    L = batch.seq_lens
    qsl = batch.query_start_loc
    B = len(L)
    seqs = set(rng.choice(B, size=min(B, max_seqs), replace=False).tolist())
    seqs.add(int(np.argmax(L)))
    seqs.add(int(np.argmin(L)))
    rows = []
    for b in sorted(seqs):
        r0, r1 = int(qsl[b]), int(qsl[b + 1])
        n = r1 - r0
        pick = {0, n - 1}
        if n > 2:
            pick.update(rng.choice(np.arange(1, n - 1), size=min(per_seq, n - 2), replace=False).tolist())
        rows.extend(r0 + i for i in sorted(pick))
    return np.array(sorted(set(rows)), dtype=np.int64)
