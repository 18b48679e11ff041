"""The HND memory order of the pool and large pages (128 .. 1024 tokens) on the
GPU, through the C ABI, against the CPU oracle; the memory order must not
change a single output bit."""
import numpy as np
import pytest

import attention_paged_kv_varlen_amd as pa
import oracle
from tests.gpu_helpers import announce, assert_close, oracle_full, run_gpu
from workloads import f32_to_bf16_bits, make_batch

pytestmark = pytest.mark.gpu

MIXED = dict(qlens=[1, 1, 1, 1, 37, 130, 200], lens=[1, 17, 700, 2100, 337, 130, 1300])

CASES = {
    "bf16_d128_g4_bs16": dict(num_heads=8, num_kv_heads=2, head_size=128, block_size=16),
    "bf16_d128_g8_bs64": dict(num_heads=16, num_kv_heads=2, head_size=128, block_size=64),
    "bf16_d64_g2_bs32": dict(num_heads=4, num_kv_heads=2, head_size=64, block_size=32),
    "fp32_d128_g2_bs16": dict(num_heads=4, num_kv_heads=2, head_size=128, block_size=16, dtype="fp32"),
    "e4m3_d128_g4_bs16": dict(num_heads=8, num_kv_heads=2, head_size=128, block_size=16, kv_dtype="fp8_e4m3"),
    "bf16_d128_g4_bs128": dict(num_heads=8, num_kv_heads=2, head_size=128, block_size=128),
    "bf16_d128_g4_bs256": dict(num_heads=8, num_kv_heads=2, head_size=128, block_size=256),
    "bf16_d128_g4_bs1024": dict(num_heads=8, num_kv_heads=2, head_size=128, block_size=1024),
    "e4m3_d128_g8_bs512": dict(num_heads=16, num_kv_heads=2, head_size=128, block_size=512, kv_dtype="fp8_e4m3"),
    # pages that are not powers of two: the lookups divide, and a prefill
    # block's 16-row slabs start inside a page
    "bf16_d128_g4_bs48": dict(num_heads=8, num_kv_heads=2, head_size=128, block_size=48),
    "bf16_d128_g8_bs80": dict(num_heads=16, num_kv_heads=2, head_size=128, block_size=80),
}


@pytest.mark.parametrize("name", list(CASES))
def test_hnd_matches_oracle_and_nhd_bit_for_bit(name):
    kw = CASES[name]
    nhd = make_batch(MIXED["qlens"], MIXED["lens"], seed=60, **kw)
    hnd = make_batch(MIXED["qlens"], MIXED["lens"], seed=60, kv_layout="HND", **kw)
    announce(f"layout {name}")
    o_h, l_h, _ = run_gpu(hnd)
    ref_o, ref_l = oracle_full(hnd)
    assert_close(o_h, l_h, ref_o, ref_l, f"HND {name}")
    o_n, l_n, _ = run_gpu(nhd)
    assert_close(o_n, l_n, ref_o, ref_l, f"NHD {name}")
    assert np.array_equal(o_h, o_n) and np.array_equal(l_h, l_n), "memory order changed the result"


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_large_page_cascade(layout):
    P = 256
    qlens = [1, 1, 1, 1, 20]
    lens = [P + e for e in (5, 140, 300, 1, 20)]
    b = make_batch(qlens, lens, num_heads=8, num_kv_heads=2, head_size=128, block_size=128, seed=61,
                   shared_prefix_blocks=P // 128, kv_layout=layout)
    announce(f"cascade bs=128 {layout}")
    ref_o, ref_l = oracle_full(b)
    co, cl, _ = run_gpu(b)
    assert_close(co, cl, ref_o, ref_l, f"cascade {layout}")
    po, pl, _ = run_gpu(b, common_prefix_len=0)
    assert_close(co, cl, po, pl, f"cascade vs non-cascade {layout}")


@pytest.mark.parametrize("bs", [16, 1024])
def test_hnd_decode_only_balanced_lists(bs):
    rng = np.random.default_rng(62)
    lens = rng.integers(1, 3000, size=10).tolist() + [1, 4096]
    b = make_batch([1] * len(lens), lens, num_heads=32, num_kv_heads=8, head_size=128, block_size=bs, seed=63,
                   kv_layout="HND")
    announce(f"HND decode_only bs={bs}")
    out, lse, db = run_gpu(b)
    assert pa.pa_plan_get_info(db.plan)["decode_list_tokens"] > 0
    ref_o, ref_l = oracle_full(b)
    assert_close(out, lse, ref_o, ref_l, f"HND decode bs={bs}")


def _params(b, **kw):
    return pa.make_params(num_seqs=b.num_seqs, num_heads=b.num_heads, num_kv_heads=b.num_kv_heads,
                          head_size=b.head_size, block_size=b.block_size, num_blocks=b.kv_cache.shape[0],
                          max_blocks_per_seq=b.block_table.shape[1], dtype=b.dtype, scale=b.scale,
                          kv_layout=b.kv_layout, kv_dtype=b.kv_dtype, **kw)


@pytest.mark.parametrize("kv_dtype", ["same", "fp8_e4m3"])
def test_hnd_gather_is_bit_exact(kv_dtype):
    import torch
    b = make_batch([1, 1, 5], [40, 300, 1100], num_heads=8, num_kv_heads=2, head_size=128, block_size=256,
                   seed=64, kv_layout="HND", kv_dtype=kv_dtype)
    announce(f"HND gather {kv_dtype}")
    pool = torch.from_numpy(b.kv_cache).cuda()
    params = _params(b)
    for s in range(b.num_seqs):
        L = int(b.seq_lens[s])
        row = torch.from_numpy(b.block_table[s].copy()).cuda()
        k = torch.empty((L, b.num_kv_heads, b.head_size), dtype=pool.dtype, device="cuda")
        v = torch.empty_like(k)
        pa.pa_gather_kv(pool, row, L, params, k, v)
        torch.cuda.synchronize()
        K, V = oracle.gather(b.kv_cache, b.block_table[s], L, kv_layout="HND")
        assert np.array_equal(k.cpu().numpy(), K, equal_nan=True) and np.array_equal(v.cpu().numpy(), V, equal_nan=True)


@pytest.mark.parametrize("kv_dtype", ["same", "fp8_e4m3"])
def test_hnd_write_is_bit_exact(kv_dtype):
    import torch
    b = make_batch([1, 8, 1], [17, 40, 600], num_heads=8, num_kv_heads=2, head_size=128, block_size=128,
                   seed=65, kv_layout="HND", kv_dtype=kv_dtype)
    announce(f"HND write {kv_dtype}")
    slots = oracle.slot_mapping(b.query_start_loc, b.seq_lens, b.block_table, b.block_size)
    slots[1] = -1
    T = len(slots)
    rng = np.random.default_rng(66)
    kb = f32_to_bf16_bits(rng.standard_normal((T, b.num_kv_heads, b.head_size)).astype(np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((T, b.num_kv_heads, b.head_size)).astype(np.float32))
    pool = torch.from_numpy(b.kv_cache.copy()).cuda()
    tk = torch.from_numpy(kb).view(torch.bfloat16).cuda()
    tv = torch.from_numpy(vb).view(torch.bfloat16).cuda()
    ts = torch.from_numpy(slots).cuda()
    if kv_dtype == "same":
        pa.pa_write_kv(tk, tv, ts, T, _params(b), pool)
        want = oracle.write_kv(b.kv_cache, kb, vb, slots, kv_layout="HND")
    else:
        pa.pa_write_kv_fp8(tk, tv, ts, T, _params(b), torch.from_numpy(b.k_scale).cuda(),
                           torch.from_numpy(b.v_scale).cuda(), pool)
        want = oracle.write_kv_fp8(b.kv_cache, oracle.to_f64(kb, "bf16"), oracle.to_f64(vb, "bf16"), slots,
                                   b.k_scale, b.v_scale, kv_layout="HND")
    torch.cuda.synchronize()
    got = pool.cpu().numpy()
    assert got.view(np.uint8).tobytes() == np.ascontiguousarray(want).view(np.uint8).tobytes()
