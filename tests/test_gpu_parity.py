"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Small batches are compared on every element; the full-size workloads on every
row (decode-only, chunked-prefill mixed, cascade) or a dense spread of rows of
every prompt (causal varlen prefill), plus properties that hold at any size
(finite outputs, cascade = non-cascade).  Gathers are bit-exact.
"""
import numpy as np
import pytest

import attention_paged_kv_varlen_amd as pa
import oracle
from tests.gpu_helpers import LSE_TOL, OUT_TOL, announce, assert_close, oracle_full, run_gpu
from workloads import config_batch, f32_to_bf16_bits, make_batch

pytestmark = pytest.mark.gpu


def _mixed(qlens, lens, **kw):
    return lambda: make_batch(qlens, lens, **kw)


SMALL = {
    # configuration 1 exactly: fp32, 2 decodes, a chunk with 48 context tokens, a full prefill
    "cfg1_tiny_mixed_fp32": lambda: config_batch(1),
    "mixed_bf16_d128_g4_bs16": _mixed([1, 1, 1, 1, 1, 37, 130, 200], [1, 16, 17, 700, 2100, 337, 130, 264],
                                      num_heads=8, num_kv_heads=2, head_size=128, block_size=16, seed=11),
    "mixed_bf16_d128_g8_bs64": _mixed([1, 1, 1, 64, 100, 1], [65, 640, 1500, 600, 100, 64],
                                      num_heads=16, num_kv_heads=2, head_size=128, block_size=64, seed=12),
    "mixed_bf16_d64_g2_bs32": _mixed([1, 1, 33, 70, 1], [5, 333, 100, 70, 1000],
                                     num_heads=4, num_kv_heads=2, head_size=64, block_size=32, seed=13),
    "mixed_fp32_d128_g1_bs16": _mixed([1, 1, 150, 20], [40, 513, 150, 300],
                                      num_heads=2, num_kv_heads=2, head_size=128, block_size=16, dtype="fp32",
                                      seed=14),
    "mixed_fp32_d64_g4_bs16": _mixed([1, 17, 1], [90, 17, 33],
                                     num_heads=8, num_kv_heads=2, head_size=64, block_size=16, dtype="fp32",
                                     seed=15),
    "mixed_bf16_d128_g16_bs16": _mixed([1, 1, 40, 1], [300, 1, 90, 47],
                                       num_heads=16, num_kv_heads=1, head_size=128, block_size=16, seed=16),
    "mixed_bf16_d128_g32_bs48": _mixed([1, 1, 50], [700, 49, 150],
                                       num_heads=32, num_kv_heads=1, head_size=128, block_size=48, seed=17),
    "mixed_bf16_d128_g3_bs16": _mixed([1, 30, 1], [77, 95, 1200],
                                      num_heads=6, num_kv_heads=2, head_size=128, block_size=16, seed=18),
    "noncausal_bf16_d128_g4": _mixed([1, 40, 7], [64, 100, 7], num_heads=8, num_kv_heads=2, head_size=128,
                                     block_size=16, seed=19, causal=False),
    # page sizes that are not powers of two take the division path of the
    # page lookups in the general prefill kernel too
    "mixed_bf16_d64_g2_bs80": _mixed([1, 45, 1, 90], [300, 45, 81, 250],
                                     num_heads=4, num_kv_heads=2, head_size=64, block_size=80, seed=20),
    "mixed_fp32_d128_g2_bs48": _mixed([1, 33, 1], [100, 130, 49],
                                      num_heads=4, num_kv_heads=2, head_size=128, block_size=48, dtype="fp32",
                                      seed=21),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_batch_matches_oracle(name):
    batch = SMALL[name]()
    announce(f"{name} B={batch.num_seqs} T={batch.num_tokens} H={batch.num_heads}/{batch.num_kv_heads} "
             f"d={batch.head_size} bs={batch.block_size} {batch.dtype} causal={batch.causal}")
    out, lse, _ = run_gpu(batch)
    ref_o, ref_l = oracle_full(batch)
    assert_close(out, lse, ref_o, ref_l, name)


# Decodes beside prefills with 4 and 8 KV heads over a bf16 pool, head size
# 128: the 8-wave wide prefill on the side stream beside 8-wave (Hkv = 8) or
# 4-wave (Hkv = 4) decode workgroups.  Ragged prompts, chunks with context,
# non-causal rows, HND order and 64- and 128-token pages.
WIDE_HKV = {
    "hkv8_g4_bs16": ([1, 1, 1, 1, 1, 37, 130, 200], [1, 16, 17, 700, 2100, 337, 130, 264],
                     dict(num_heads=32, num_kv_heads=8, block_size=16)),
    "hkv4_g8_bs64": ([1, 1, 1, 64, 100, 1], [65, 640, 1500, 600, 100, 64],
                     dict(num_heads=32, num_kv_heads=4, block_size=64)),
    "hkv4_g2_noncausal": ([1, 40, 7, 1], [64, 100, 7, 999], dict(num_heads=8, num_kv_heads=4, block_size=16,
                                                                  causal=False)),
    "hkv8_g8_hnd_bs128": ([1, 1, 300, 1, 17], [4000, 129, 2300, 1, 17],
                          dict(num_heads=64, num_kv_heads=8, block_size=128, kv_layout="HND")),
}


@pytest.mark.parametrize("name", list(WIDE_HKV))
def test_decodes_beside_wide_prefill_match_oracle(name):
    qlens, lens, kw = WIDE_HKV[name]
    batch = make_batch(qlens, lens, head_size=128, seed=61, **kw)
    announce(f"wide hkv {name} B={batch.num_seqs} T={batch.num_tokens}")
    out, lse, db = run_gpu(batch)
    info = pa.pa_plan_get_info(db.plan)
    assert info["num_decode_items"] > 0 and info["num_prefill_items"] > 0
    ref_o, ref_l = oracle_full(batch)
    assert_close(out, lse, ref_o, ref_l, f"wide hkv {name}")


# Batches of decodes alone with the automatic split: balanced work lists that
# cross sequence boundaries, under every decode launch shape (waves per
# workgroup = the largest divisor of Hkv x ceil(g / 16) up to 8).
DECODE_ONLY = {
    "g4_hkv2_bs16": dict(num_heads=8, num_kv_heads=2, head_size=128, block_size=16),
    "g8_hkv8_bs64": dict(num_heads=64, num_kv_heads=8, head_size=128, block_size=64),
    "g1_hkv6_bs48": dict(num_heads=6, num_kv_heads=6, head_size=128, block_size=48),
    "g32_hkv1_bs16": dict(num_heads=32, num_kv_heads=1, head_size=128, block_size=16),
    "g3_hkv3_d64": dict(num_heads=9, num_kv_heads=3, head_size=64, block_size=32),
    "g2_hkv4_fp32": dict(num_heads=8, num_kv_heads=4, head_size=128, block_size=16, dtype="fp32"),
}


@pytest.mark.parametrize("name", list(DECODE_ONLY))
def test_decode_only_balanced_lists_match_oracle(name):
    rng = np.random.default_rng(31)
    lens = rng.integers(1, 1500, size=9).tolist() + [1, 33, 2048]
    batch = make_batch([1] * len(lens), lens, seed=32, **DECODE_ONLY[name])
    announce(f"decode_only {name} B={batch.num_seqs}")
    out, lse, db = run_gpu(batch)
    info = pa.pa_plan_get_info(db.plan)
    assert info["decode_list_tokens"] > 0 and info["num_decode_lists"] < info["num_decode_items"]
    ref_o, ref_l = oracle_full(batch)
    assert_close(out, lse, ref_o, ref_l, name)


def test_cascade_small_matches_oracle_and_non_cascade():
    P = 128
    qlens = [1, 1, 1, 1, 1, 1, 20, 9]
    extra = [5, 40, 100, 1, 300, 17, 70, 9]
    lens = [P + e for e in extra]
    batch = make_batch(qlens, lens, num_heads=8, num_kv_heads=2, head_size=128, block_size=16, seed=21,
                       shared_prefix_blocks=P // 16)
    announce(f"cascade_small P={P} B={batch.num_seqs}")
    ref_o, ref_l = oracle_full(batch)
    co, cl, _ = run_gpu(batch)
    assert_close(co, cl, ref_o, ref_l, "cascade vs oracle")
    po, pl, _ = run_gpu(batch, common_prefix_len=0)
    assert_close(po, pl, ref_o, ref_l, "non-cascade vs oracle")
    assert_close(co, cl, po, pl, "cascade vs non-cascade")


# A shared prefix with decodes alone: the prefix pass, then balanced decode
# lists over the suffixes (starting at P), then the merge.  Pieces of a list may
# start off a 32-key boundary of the sequence (P = 16 x odd), pages may hold
# 128 keys in HND order, and the pool may hold e4m3 codes.
CASCADE_DECODES = {
    "bf16_bs16_P128": dict(P=128, block_size=16),
    "bf16_bs16_P16x21": dict(P=16 * 21, block_size=16),
    "fp32_bs16_P64": dict(P=64, block_size=16, dtype="fp32"),
    "bf16_hnd_bs128_P256": dict(P=256, block_size=128, kv_layout="HND"),
    "e4m3_bs16_P144": dict(P=144, block_size=16, kv_dtype="fp8_e4m3"),
    "bf16_g8_bs64_P192": dict(P=192, block_size=64, num_heads=16),
    # 8 KV heads: 8-wave decode workgroups, so the prefix pass runs in the
    # decode's own launch (prefix_decode_kernel), on CUs of its own
    "fused_hkv8_bs16_P16x37": dict(P=16 * 37, block_size=16, num_heads=32, num_kv_heads=8),
    "fused_hkv8_hnd_bs128_P1024": dict(P=1024, block_size=128, num_heads=32, num_kv_heads=8, kv_layout="HND"),
    "fused_hkv8_g8_bs64_P2048": dict(P=2048, block_size=64, num_heads=64, num_kv_heads=8),
}


@pytest.mark.parametrize("name", list(CASCADE_DECODES))
def test_cascade_decodes_only_match_oracle(name):
    kw = dict(CASCADE_DECODES[name])
    P = kw.pop("P")
    kw.setdefault("num_heads", 8)
    kw.setdefault("num_kv_heads", 2)
    rng = np.random.default_rng(23)
    extra = rng.integers(1, 900, size=14).tolist() + [1, 31, 33, 1000]
    lens = [P + e for e in extra]
    batch = make_batch([1] * len(lens), lens, head_size=128, seed=24, shared_prefix_blocks=P // kw["block_size"],
                       **kw)
    announce(f"cascade decodes only {name} B={batch.num_seqs} P={P}")
    co, cl, db = run_gpu(batch)
    info = pa.pa_plan_get_info(db.plan)
    assert info["num_prefill_items"] == 0 and info["num_prefix_items"] > 0
    fused = name.startswith("fused")
    assert info["prefix_beside_decode"] == (1 if fused else 0)
    assert 0 < info["num_decode_lists"] < info["num_decode_items"] and info["decode_list_tokens"] > 0
    ref_o, ref_l = oracle_full(batch)
    assert_close(co, cl, ref_o, ref_l, f"{name} cascade vs oracle")
    po, pl, _ = run_gpu(batch, common_prefix_len=0)
    assert_close(po, pl, ref_o, ref_l, f"{name} non-cascade vs oracle")


@pytest.mark.parametrize("split", [32, 96, 512, 0])
def test_split_kv_invariance(split):
    rng = np.random.default_rng(22)
    lens = rng.integers(1, 3000, size=12).tolist() + [4096, 33]
    batch = make_batch([1] * len(lens), lens, num_heads=8, num_kv_heads=2, head_size=128, block_size=16, seed=22)
    announce(f"split_kv split={split}")
    ref_o, ref_l = oracle_full(batch)
    out, lse, db = run_gpu(batch, kv_split_tokens=split)
    if split == 0:  # decodes alone, automatic split: balanced lists, some items share a list
        info = pa.pa_plan_get_info(db.plan)
        assert info["decode_list_tokens"] > 0 and info["num_decode_lists"] < info["num_decode_items"]
    assert_close(out, lse, ref_o, ref_l, f"split {split}")
    base_o, base_l, _ = run_gpu(batch, kv_split_tokens=4096)
    assert_close(out, lse, base_o, base_l, f"split {split} vs one split")


def test_block_permutation_is_bit_exact():
    batch = SMALL["mixed_bf16_d128_g4_bs16"]()
    announce("block_permutation")
    o1, l1, _ = run_gpu(batch)
    rng = np.random.default_rng(23)
    perm = rng.permutation(batch.num_blocks)
    pool2 = np.empty_like(batch.kv_cache)
    pool2[perm] = batch.kv_cache
    bt2 = perm[batch.block_table].astype(np.int32)
    o2, l2, _ = run_gpu(batch, kv_cache=pool2, block_table=bt2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_runs_are_deterministic():
    batch = SMALL["mixed_bf16_d128_g8_bs64"]()
    announce("determinism")
    o1, l1, db = run_gpu(batch, kv_split_tokens=64)
    import torch
    db.forward()
    torch.cuda.synchronize()
    o2 = db.out.float().cpu().numpy().astype(np.float64)
    l2 = db.lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_gather_is_bit_exact():
    import torch

    import attention_paged_kv_varlen_amd as pa
    for name in ("mixed_bf16_d128_g8_bs64", "mixed_fp32_d128_g1_bs16", "mixed_bf16_d64_g2_bs32"):
        batch = SMALL[name]()
        announce(f"gather {name}")
        db = pa.to_device(batch.q, batch.kv_cache, batch.block_table, batch.query_start_loc, batch.seq_lens,
                          num_heads=batch.num_heads, num_kv_heads=batch.num_kv_heads, head_size=batch.head_size,
                          block_size=batch.block_size, dtype=batch.dtype, scale=batch.scale)
        tdt = torch.bfloat16 if batch.dtype == "bf16" else torch.float32
        for b in range(batch.num_seqs):
            L = int(batch.seq_lens[b])
            k = torch.empty((L, batch.num_kv_heads, batch.head_size), dtype=tdt, device="cuda")
            v = torch.empty_like(k)
            pa.pa_gather_kv(db.kv_cache, db.block_table[b], L, db.params, k, v)
            torch.cuda.synchronize()
            K, V = oracle.gather(batch.kv_cache, batch.block_table[b], L)
            view = torch.uint16 if batch.dtype == "bf16" else torch.int32
            kb = k.view(view).cpu().numpy()
            vb = v.view(view).cpu().numpy()
            assert np.array_equal(kb, K.view(kb.dtype)) and np.array_equal(vb, V.view(vb.dtype))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_merge_states_matches_oracle(dtype):
    import torch

    import attention_paged_kv_varlen_amd as pa
    announce(f"merge_states {dtype}")
    rng = np.random.default_rng(24)
    T, H, D = 37, 6, 128
    oa = rng.standard_normal((T, H, D)).astype(np.float32)
    ob = rng.standard_normal((T, H, D)).astype(np.float32)
    la = (rng.standard_normal((T, H)) * 5).astype(np.float32)
    lb = (rng.standard_normal((T, H)) * 5).astype(np.float32)
    la[0, 0] = -np.inf
    lb[1, 1] = -np.inf
    la[2, 2] = lb[2, 2] = -np.inf
    if dtype == "bf16":
        oa_h, ob_h = f32_to_bf16_bits(oa), f32_to_bf16_bits(ob)
        ta = torch.from_numpy(oa_h).view(torch.bfloat16).cuda()
        tb = torch.from_numpy(ob_h).view(torch.bfloat16).cuda()
    else:
        oa_h, ob_h = oa, ob
        ta, tb = torch.from_numpy(oa).cuda(), torch.from_numpy(ob).cuda()
    tla, tlb = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    to = torch.empty_like(ta)
    tl = torch.empty_like(tla)
    pa.pa_merge_states(ta, tla, tb, tlb, to, tl)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge_states(oracle.to_f64(oa_h, dtype), la, oracle.to_f64(ob_h, dtype), lb)
    got_o = to.float().cpu().numpy().astype(np.float64)
    got_l = tl.cpu().numpy().astype(np.float64)
    both = np.isinf(ref_l)
    assert np.array_equal(np.isinf(got_l), both)
    assert np.max(np.abs(got_o - ref_o)) <= OUT_TOL
    assert np.max(np.abs(got_l[~both] - ref_l[~both])) <= LSE_TOL
    assert np.all(got_o[both] == 0)


def test_gpu_closed_forms():
    """q = 0 gives the mean of the visible V rows and LSE = ln(count); a single
    key gives its V row exactly; the ramp needle picks V[c + i]."""
    qlens, lens = [1, 1, 1, 16, 40], [1, 17, 250, 64, 40]
    batch = make_batch(qlens, lens, num_heads=8, num_kv_heads=2, head_size=128, block_size=16, seed=25)
    announce("closed_forms equal scores")
    q0 = np.zeros_like(batch.q)
    out, lse, _ = run_gpu(batch, q=q0)
    qsl = batch.query_start_loc
    for b, (qb, L) in enumerate(zip(qlens, lens)):
        for i in range(qb):
            n = L - qb + i + 1
            assert np.max(np.abs(lse[qsl[b] + i] - np.log(n))) <= LSE_TOL
    ref_o, ref_l = oracle_full(batch, q=q0)
    assert_close(out, lse, ref_o, ref_l, "equal scores")
    # single key: the sequence of length 1 returns V[0] bit for bit
    K, V = oracle.gather(batch.kv_cache, batch.block_table[0], 1)
    got = run_gpu(batch)[0][0]
    assert np.array_equal(got, np.repeat(oracle.to_f64(V[0], "bf16"), 4, axis=0))
    # ramp needle: K[t, :, 0] = 256 t, q[., 0] = 1
    announce("closed_forms ramp needle")
    pool = batch.kv_cache.copy()
    bs = batch.block_size
    for b, L in enumerate(lens):
        for t in range(L):
            blk = batch.block_table[b, t // bs]
            pool[blk, 0, t % bs] = 0
            pool[blk, 0, t % bs, :, 0] = f32_to_bf16_bits(np.array([256.0 * t], np.float32))[0]
    qn = np.zeros_like(batch.q)
    qn[:, :, 0] = f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    out, lse, _ = run_gpu(batch, q=qn, kv_cache=pool)
    for b, (qb, L) in enumerate(zip(qlens, lens)):
        _, Vb = oracle.gather(pool, batch.block_table[b], L)
        for i in range(qb):
            want = np.repeat(oracle.to_f64(Vb[L - qb + i], "bf16"), 4, axis=0)
            assert np.max(np.abs(out[qsl[b] + i] - want)) <= OUT_TOL


def test_forward_rejects_small_workspace_and_keeps_outputs():
    import torch

    import attention_paged_kv_varlen_amd as pa
    batch = SMALL["mixed_bf16_d128_g4_bs16"]()
    announce("workspace too small")
    db = pa.to_device(batch.q, batch.kv_cache, batch.block_table, batch.query_start_loc, batch.seq_lens,
                      num_heads=batch.num_heads, num_kv_heads=batch.num_kv_heads, head_size=batch.head_size,
                      block_size=batch.block_size, dtype=batch.dtype, scale=batch.scale, kv_split_tokens=64)
    need = pa.pa_plan_workspace_bytes(db.plan)
    assert need > 0
    db.out.fill_(3.0)
    with pytest.raises(pa.PagedAttnError) as ei:
        pa.pa_forward(db.plan, db.q, db.kv_cache, db.block_table, db.query_start_loc, db.seq_lens, db.out, db.lse,
                      db.workspace, workspace_bytes=need - 1)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert bool(torch.all(db.out.float() == 3.0))


def test_profile_records_kernel_times():
    import torch

    import attention_paged_kv_varlen_amd as pa
    batch = SMALL["mixed_bf16_d128_g4_bs16"]()
    announce("profile")
    db = pa.to_device(batch.q, batch.kv_cache, batch.block_table, batch.query_start_loc, batch.seq_lens,
                      num_heads=batch.num_heads, num_kv_heads=batch.num_kv_heads, head_size=batch.head_size,
                      block_size=batch.block_size, dtype=batch.dtype, scale=batch.scale, kv_split_tokens=64)
    pa.pa_profile_start(16)
    db.forward()
    db.forward()
    rec = pa.pa_profile_stop()
    torch.cuda.synchronize()
    names = {r["name"]: r for r in rec}
    assert "decode_bf16_d128" in names and "prefill_bf16_d128" in names and "merge_bf16_d128" in names
    assert all(r["launches"] == 2 and r["total_ms"] > 0 for r in rec)


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

def full_config_rows(batch, cfg):
    """Rows of a full-size workload compared with the oracle: every row of the
    decode-only, chunked-prefill mixed and cascade workloads and of the cascade
    with chunks (the oracle takes seconds for them), and for the causal varlen prefill (1.7 TFLOP of dense
    float64 work in all) the first and last 8 rows of every prompt plus 48
    spread between them (so every prompt's first, middle and last tiles and
    its ragged tail are covered)."""
    qsl = batch.query_start_loc
    if cfg != 3:
        return np.arange(int(qsl[-1]), dtype=np.int64)
    rows = []
    for b in range(batch.num_seqs):
        r0, r1 = int(qsl[b]), int(qsl[b + 1])
        rows += list(range(r0, min(r0 + 8, r1))) + list(range(max(r0, r1 - 8), r1))
        rows += np.linspace(r0, r1 - 1, 48).astype(np.int64).tolist()
    return np.array(sorted(set(rows)), dtype=np.int64)


def _row_kinds(batch, rows):
    ql = np.diff(batch.query_start_loc)
    seq = np.searchsorted(batch.query_start_loc, rows, side="right") - 1
    dec = ql[seq] == 1
    return int(dec.sum()), int((~dec).sum()), len(np.unique(seq[~dec]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3, 4, 6])
def test_full_config_against_oracle(cfg):
    announce(f"full config {cfg}: generating")
    batch = config_batch(cfg)
    announce(f"full config {cfg}: B={batch.num_seqs} T={batch.num_tokens} pool={batch.kv_cache.nbytes / 1e9:.2f} GB")
    out, lse, _ = run_gpu(batch)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    rows = full_config_rows(batch, cfg)
    n_dec, n_pre, n_pre_seqs = _row_kinds(batch, rows)
    announce(f"full config {cfg}: comparing {len(rows)} of {batch.num_tokens} rows with the oracle "
             f"({n_dec} decode rows, {n_pre} prefill rows of {n_pre_seqs} sequences)")
    if cfg in (4, 6):  # all four chunks, every row
        assert n_pre == 4 * 512 and n_pre_seqs == 4
    ref_o, ref_l = oracle.attention_rows(batch.q, batch.kv_cache, batch.block_table, batch.query_start_loc,
                                         batch.seq_lens, batch.scale, rows, dtype=batch.dtype)
    assert_close(out[rows], lse[rows], ref_o, ref_l, f"config {cfg} ({len(rows)} rows)")


@pytest.mark.timeout(900)
def test_full_config5_cascade():
    announce("full config 5: generating")
    batch = config_batch(5)
    announce(f"full config 5: B={batch.num_seqs} P={batch.common_prefix_len}")
    co, cl, db = run_gpu(batch)
    info = pa.pa_plan_get_info(db.plan)
    assert info["common_prefix_len"] == batch.common_prefix_len and info["num_prefix_items"] > 0
    po, pl, _ = run_gpu(batch, common_prefix_len=0)
    assert_close(co, cl, po, pl, "config 5 cascade vs non-cascade (all rows)")
    rows = full_config_rows(batch, 5)
    announce(f"full config 5: comparing all {len(rows)} rows (cascade and non-cascade) with the oracle")
    ref_o, ref_l = oracle.attention_rows(batch.q, batch.kv_cache, batch.block_table, batch.query_start_loc,
                                         batch.seq_lens, batch.scale, rows, dtype=batch.dtype)
    assert_close(co[rows], cl[rows], ref_o, ref_l, f"config 5 cascade ({len(rows)} rows)")
    assert_close(po[rows], pl[rows], ref_o, ref_l, f"config 5 non-cascade ({len(rows)} rows)")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_write_kv_is_bit_exact(dtype):
    """Random tokens into a NaN-poisoned pool: the pool after pa_write_kv equals
    the oracle's write_kv bit for bit; negative and out-of-pool slots are skipped."""
    import torch
    announce(f"write_kv {dtype}")
    rng = np.random.default_rng(41)
    nb, bs, Hkv, d, T = 40, 16, 4, 128, 300
    shape = (nb, 2, bs, Hkv, d)
    if dtype == "bf16":
        pool = np.full(shape, 0x7FC0, dtype=np.uint16)
        k = f32_to_bf16_bits(rng.standard_normal((T, Hkv, d)).astype(np.float32))
        v = f32_to_bf16_bits(rng.standard_normal((T, Hkv, d)).astype(np.float32))
    else:
        pool = np.full(shape, np.nan, dtype=np.float32)
        k = rng.standard_normal((T, Hkv, d)).astype(np.float32)
        v = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)  # distinct slots
    slots[::17] = -1
    slots[5] = nb * bs + 3  # past the pool: skipped
    want = oracle.write_kv(pool, k, v, np.where(slots >= nb * bs, -1, slots))

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.int16) if a.dtype == np.uint16 else t).to("cuda:0")
    tp, tk, tv, ts = dev(pool), dev(k), dev(v), dev(slots)
    params = pa.make_params(num_seqs=1, num_heads=Hkv, num_kv_heads=Hkv, head_size=d, block_size=bs, num_blocks=nb,
                            max_blocks_per_seq=1, dtype=dtype, scale=0.1)
    pa.pa_write_kv(tk, tv, ts, T, params, tp)
    torch.cuda.synchronize()
    got = tp.cpu().numpy()
    if dtype == "bf16":
        assert np.array_equal(got.view(np.uint16), want)
    else:
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_write_kv_then_attention_matches_oracle():
    """The new tokens of a mixed batch, erased from the pool and written back
    through the slot mapping with pa_write_kv, give back the same pool and the
    oracle's attention."""
    import torch
    batch = SMALL["mixed_bf16_d128_g4_bs16"]()
    announce("write_kv then attention")
    slots = oracle.slot_mapping(batch.query_start_loc, batch.seq_lens, batch.block_table, batch.block_size)
    T = batch.num_tokens
    Hkv, d, bs = batch.num_kv_heads, batch.head_size, batch.block_size
    k = np.empty((T, Hkv, d), dtype=np.uint16)
    v = np.empty((T, Hkv, d), dtype=np.uint16)
    erased = batch.kv_cache.copy()
    for t, s in enumerate(slots):
        k[t], v[t] = batch.kv_cache[s // bs, 0, s % bs], batch.kv_cache[s // bs, 1, s % bs]
        erased[s // bs, :, s % bs] = 0x7FC0
    tp = torch.from_numpy(erased).view(torch.int16).to("cuda:0")
    params = pa.make_params(num_seqs=batch.num_seqs, num_heads=batch.num_heads, num_kv_heads=Hkv, head_size=d,
                            block_size=bs, num_blocks=batch.num_blocks, max_blocks_per_seq=batch.max_blocks_per_seq,
                            dtype="bf16", scale=batch.scale)
    pa.pa_write_kv(torch.from_numpy(k).view(torch.int16).to("cuda:0"), torch.from_numpy(v).view(torch.int16).to("cuda:0"),
                   torch.from_numpy(slots).to("cuda:0"), T, params, tp)
    torch.cuda.synchronize()
    assert np.array_equal(tp.cpu().numpy().view(np.uint16), batch.kv_cache)
    out, lse, _ = run_gpu(batch, kv_cache=tp.cpu().numpy().view(np.uint16))
    ref_o, ref_l = oracle_full(batch)
    assert_close(out, lse, ref_o, ref_l, "write_kv then attention")
