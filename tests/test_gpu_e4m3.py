"""The e4m3 (8-bit float) KV cache on the GPU, through the C ABI, against the
CPU oracle: conversion of every code, mixed / decode-only / cascade batches,
the byte-exact gather, and the quantising cache write (bit-exact codes)."""
import numpy as np
import pytest

import attention_paged_kv_varlen_amd as pa
import oracle
from tests.gpu_helpers import announce, assert_close, oracle_full, run_gpu
from workloads import config_batch, f32_to_bf16_bits, make_batch

pytestmark = pytest.mark.gpu


def _f8(qlens, lens, **kw):
    return lambda: make_batch(qlens, lens, kv_dtype="fp8_e4m3", **kw)


def test_every_code_widens_exactly():
    # One sequence with a single key: the output is that key's V row times the
    # V scale.  The V rows of the two KV heads hold all 256 codes (0..127 and
    # 128..255); power-of-two scales keep every product exact in bf16, so the
    # output must equal the oracle's decoded values exactly, NaN at 0x7F / 0xFF.
    announce("e4m3 every code")
    b = make_batch([1], [1], num_heads=2, num_kv_heads=2, head_size=128, block_size=16, seed=40,
                   kv_dtype="fp8_e4m3")
    kv = b.kv_cache.copy()
    blk = int(b.block_table[0, 0])
    kv[blk, 1, 0, 0] = np.arange(128, dtype=np.uint8)
    kv[blk, 1, 0, 1] = np.arange(128, 256, dtype=np.uint8)
    kv[blk, 0, 0] = np.where(kv[blk, 0, 0] & 0x7F == 0x7F, 0x38, kv[blk, 0, 0])  # finite K
    b.kv_cache = kv
    b.k_scale = np.array([1.0, 1.0], dtype=np.float32)
    b.v_scale = np.array([0.5, 4.0], dtype=np.float32)
    out, lse, _ = run_gpu(b)
    want = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)).reshape(2, 128) * b.v_scale[:, None]
    got = out[0]
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    ref_o, ref_l = oracle_full(b)
    assert np.abs(lse - ref_l).max() < 1e-4


SMALL = {
    "mixed_d128_g4_bs16": _f8([1, 1, 1, 1, 1, 37, 130, 200], [1, 16, 17, 700, 2100, 337, 130, 264],
                              num_heads=8, num_kv_heads=2, head_size=128, block_size=16, seed=41),
    "mixed_d128_g8_bs64": _f8([1, 1, 1, 64, 100, 1], [65, 640, 1500, 600, 100, 64],
                              num_heads=16, num_kv_heads=2, head_size=128, block_size=64, seed=42),
    "mixed_d64_g2_bs32": _f8([1, 1, 33, 70, 1], [5, 333, 100, 70, 1000],
                             num_heads=4, num_kv_heads=2, head_size=64, block_size=32, seed=43),
    "mixed_d128_g32_bs48": _f8([1, 1, 50], [700, 49, 150],
                               num_heads=32, num_kv_heads=1, head_size=128, block_size=48, seed=44),
    "noncausal_d128_g4": _f8([1, 40, 7], [64, 100, 7], num_heads=8, num_kv_heads=2, head_size=128,
                             block_size=16, seed=45, causal=False),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_batch_matches_oracle(name):
    b = SMALL[name]()
    announce(f"e4m3 {name} B={b.num_seqs} T={b.num_tokens}")
    out, lse, _ = run_gpu(b)
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, name)


def test_one_scale_for_the_tensor():
    b = SMALL["mixed_d128_g4_bs16"]()
    b.k_scale = np.array([0.0061], dtype=np.float32)
    b.v_scale = np.array([0.0057], dtype=np.float32)
    announce("e4m3 per-tensor scales")
    out, lse, db = run_gpu(b)
    assert db.k_scale.numel() == 1
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, "per-tensor scales")


@pytest.mark.parametrize("heads", [(8, 2), (64, 8), (6, 6)])
def test_decode_only_balanced_lists(heads):
    rng = np.random.default_rng(46)
    lens = rng.integers(1, 1500, size=9).tolist() + [1, 33, 2048]
    b = make_batch([1] * len(lens), lens, num_heads=heads[0], num_kv_heads=heads[1], head_size=128,
                   block_size=16, seed=47, kv_dtype="fp8_e4m3")
    announce(f"e4m3 decode_only H={heads}")
    out, lse, db = run_gpu(b)
    info = pa.pa_plan_get_info(db.plan)
    assert info["decode_list_tokens"] > 0
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, f"decode_only {heads}")


def test_cascade_matches_oracle_and_non_cascade():
    P = 128
    qlens = [1, 1, 1, 1, 1, 1, 20, 9]
    lens = [P + e for e in (5, 40, 100, 1, 300, 17, 70, 9)]
    b = make_batch(qlens, lens, num_heads=8, num_kv_heads=2, head_size=128, block_size=16, seed=48,
                   shared_prefix_blocks=P // 16, kv_dtype="fp8_e4m3")
    announce("e4m3 cascade")
    ref_o, ref_l = oracle_full(b)
    co, cl, _ = run_gpu(b)
    assert_close(co, cl, ref_o, ref_l, "cascade vs oracle")
    po, pl, _ = run_gpu(b, common_prefix_len=0)
    assert_close(co, cl, po, pl, "cascade vs non-cascade")


def test_gather_copies_codes():
    import torch
    b = SMALL["mixed_d128_g4_bs16"]()
    announce("e4m3 gather")
    pool = torch.from_numpy(b.kv_cache).cuda()
    params = pa.make_params(num_seqs=b.num_seqs, num_heads=b.num_heads, num_kv_heads=b.num_kv_heads,
                            head_size=b.head_size, block_size=b.block_size, num_blocks=b.kv_cache.shape[0],
                            max_blocks_per_seq=b.block_table.shape[1], dtype="bf16", scale=b.scale,
                            kv_dtype="fp8_e4m3")
    for s in (0, 4, 7):
        L = int(b.seq_lens[s])
        row = torch.from_numpy(b.block_table[s].copy()).cuda()
        k = torch.empty((L, b.num_kv_heads, b.head_size), dtype=torch.uint8, device="cuda")
        v = torch.empty_like(k)
        pa.pa_gather_kv(pool, row, L, params, k, v)
        torch.cuda.synchronize()
        K, V = oracle.gather(b.kv_cache, b.block_table[s], L)
        assert np.array_equal(k.cpu().numpy(), K) and np.array_equal(v.cpu().numpy(), V)


def _special_values(rng, n):
    """bf16 patterns: random N(0, 2) values plus values that land on e4m3 ties,
    overflow, underflow, signed zeros and NaN after division by the scales used."""
    x = rng.standard_normal(n).astype(np.float32) * 2
    bits = f32_to_bf16_bits(x)
    special = np.array([0x0000, 0x8000, 0x7FC0, 0xFFC0, 0x4780, 0xC780, 0x3F88, 0xBF88, 0x3F90,
                        0x3A80, 0xBA80, 0x0001, 0x8001, 0x43E0, 0x43E8, 0x4400, 0xC3F0], dtype=np.uint16)
    bits[:len(special)] = special
    return bits


@pytest.mark.parametrize("num_scales", [1, 2])
def test_write_is_bit_exact(num_scales):
    import torch
    Hkv, d, bs, nb = 2, 128, 16, 12
    rng = np.random.default_rng(49)
    T = 40
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[3] = -1
    slots[5] = nb * bs + 7          # past the pool: skipped
    kb = _special_values(rng, T * Hkv * d).reshape(T, Hkv, d)
    vb = _special_values(rng, T * Hkv * d)[::-1].copy().reshape(T, Hkv, d)
    ks = np.array([1.0, 0.37], dtype=np.float32)[:num_scales]
    vs = np.array([0.5, 3.1], dtype=np.float32)[:num_scales]
    pool0 = rng.integers(0, 256, size=(nb, 2, bs, Hkv, d), dtype=np.uint8)
    announce(f"e4m3 write num_scales={num_scales}")
    params = pa.make_params(num_seqs=1, num_heads=Hkv, num_kv_heads=Hkv, head_size=d, block_size=bs,
                            num_blocks=nb, max_blocks_per_seq=nb, dtype="bf16", scale=0.1, kv_dtype="fp8_e4m3")
    dev = "cuda"
    tk = torch.from_numpy(kb).view(torch.bfloat16).to(dev)
    tv = torch.from_numpy(vb).view(torch.bfloat16).to(dev)
    pool = torch.from_numpy(pool0.copy()).to(dev)
    pa.pa_write_kv_fp8(tk, tv, torch.from_numpy(slots).to(dev), T, params, torch.from_numpy(ks).to(dev),
                       torch.from_numpy(vs).to(dev), pool)
    torch.cuda.synchronize()
    kvals = oracle.to_f64(kb, "bf16")
    vvals = oracle.to_f64(vb, "bf16")
    ok_slots = np.where(slots < nb * bs, slots, -1)
    want = oracle.write_kv_fp8(pool0, kvals, vvals, ok_slots, ks, vs)
    got = pool.cpu().numpy()
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}: " \
                          f"{got[tuple(bad[0])]:#x} vs {want[tuple(bad[0])]:#x}"


def _near_ties(rng, n, scale):
    """bf16 patterns whose float32 quotient by `scale` lies within a few ulps of
    a midpoint between two e4m3 values (where the code depends on the last bit
    of the quotient), of either sign, plus values far past the saturation
    point and below the smallest e4m3 step."""
    vals = np.sort(oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    base = f32_to_bf16_bits((mids * np.float64(scale)).astype(np.float32)).astype(np.int64)
    cand = np.concatenate([base + k for k in (-2, -1, 0, 1, 2)])
    cand = np.concatenate([cand, cand | 0x8000, f32_to_bf16_bits(np.array([1e30, -1e30, 3e-38, -3e-38, 1e-40],
                                                                              dtype=np.float32)).astype(np.int64)])
    return rng.choice(cand, size=n).astype(np.uint16)


@pytest.mark.parametrize("scales", [(0.37, 3.1), (1.0 / 3.0, 7.77), (0.1, 1.7e-3), (1e-40, 2.0e38)])
def test_write_near_ties_is_bit_exact(scales):
    """The quotient by the scale decides the code near e4m3 midpoints: every
    code matches the oracle's float32 division (also for a subnormal scale
    and one whose reciprocal is subnormal)."""
    import torch
    Hkv, d, bs, nb, T = 2, 128, 16, 8, 64
    rng = np.random.default_rng(50)
    ks = np.array(scales, dtype=np.float32)
    vs = np.array(scales[::-1], dtype=np.float32)
    kb = np.stack([_near_ties(rng, T * d, ks[h]).reshape(T, d) for h in range(Hkv)], axis=1)
    vb = np.stack([_near_ties(rng, T * d, vs[h]).reshape(T, d) for h in range(Hkv)], axis=1)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    pool0 = np.zeros((nb, 2, bs, Hkv, d), dtype=np.uint8)
    announce(f"e4m3 write near ties scales={scales}")
    params = pa.make_params(num_seqs=1, num_heads=Hkv, num_kv_heads=Hkv, head_size=d, block_size=bs,
                            num_blocks=nb, max_blocks_per_seq=nb, dtype="bf16", scale=0.1, kv_dtype="fp8_e4m3")
    pool = torch.from_numpy(pool0.copy()).cuda()
    pa.pa_write_kv_fp8(torch.from_numpy(kb).view(torch.bfloat16).cuda(), torch.from_numpy(vb).view(torch.bfloat16).cuda(),
                       torch.from_numpy(slots).cuda(), T, params, torch.from_numpy(ks).cuda(),
                       torch.from_numpy(vs).cuda(), pool)
    torch.cuda.synchronize()
    want = oracle.write_kv_fp8(pool0, oracle.to_f64(kb, "bf16"), oracle.to_f64(vb, "bf16"), slots, ks, vs)
    got = pool.cpu().numpy()
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}: " \
                          f"{got[tuple(bad[0])]:#x} vs {want[tuple(bad[0])]:#x}"


def test_write_then_attention_matches_oracle():
    import torch
    b = SMALL["mixed_d128_g4_bs16"]()
    announce("e4m3 write then attention")
    qsl, L = b.query_start_loc, b.seq_lens
    slots = oracle.slot_mapping(qsl, L, b.block_table, b.block_size)
    T = len(slots)
    rng = np.random.default_rng(50)
    kb = f32_to_bf16_bits(rng.standard_normal((T, b.num_kv_heads, b.head_size)).astype(np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((T, b.num_kv_heads, b.head_size)).astype(np.float32))
    params = pa.make_params(num_seqs=b.num_seqs, num_heads=b.num_heads, num_kv_heads=b.num_kv_heads,
                            head_size=b.head_size, block_size=b.block_size, num_blocks=b.kv_cache.shape[0],
                            max_blocks_per_seq=b.block_table.shape[1], dtype="bf16", scale=b.scale,
                            kv_dtype="fp8_e4m3")
    pool = torch.from_numpy(b.kv_cache.copy()).cuda()
    pa.pa_write_kv_fp8(torch.from_numpy(kb).view(torch.bfloat16).cuda(), torch.from_numpy(vb).view(torch.bfloat16).cuda(),
                       torch.from_numpy(slots).cuda(), T, params, torch.from_numpy(b.k_scale).cuda(),
                       torch.from_numpy(b.v_scale).cuda(), pool)
    torch.cuda.synchronize()
    written = oracle.write_kv_fp8(b.kv_cache, oracle.to_f64(kb, "bf16"), oracle.to_f64(vb, "bf16"), slots,
                                  b.k_scale, b.v_scale)
    assert np.array_equal(pool.cpu().numpy(), written)
    b.kv_cache = written
    out, lse, _ = run_gpu(b)
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, "write then attention")


@pytest.mark.timeout(900)
def test_full_decode_config_all_rows():
    # the 256-sequence decode batch over an e4m3 pool, launched as the bench
    # does; every row against the oracle
    b = config_batch(2, kv_dtype="fp8_e4m3")
    announce("e4m3 full decode batch")
    out, lse, _ = run_gpu(b)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    rows = np.arange(b.num_tokens)
    announce(f"e4m3 full decode batch: comparing all {len(rows)} rows with the oracle")
    ro, rl = oracle.attention_rows(b.q, b.kv_cache, b.block_table, b.query_start_loc, b.seq_lens, b.scale, rows,
                                   kv_dtype="fp8_e4m3", k_scale=b.k_scale, v_scale=b.v_scale)
    assert_close(out[rows], lse[rows], ro, rl, "e4m3 decode batch, all rows")
