"""The host metadata builder (pa_plan_create with device < 0) on the CPU:
bit-exact agreement with the oracle's metadata, every validation error, and
the cascade read counts against the pages' read model."""
import numpy as np
import pytest

import attention_paged_kv_varlen_amd as pa
import oracle
from workloads import config_lengths


def host_plan(qlens, lens, *, H=8, Hkv=2, d=128, bs=16, dtype="bf16", block_table=None, prefix=0, split=0,
              num_blocks=None, mbs=None, causal=True):
    qlens = np.asarray(qlens)
    lens = np.asarray(lens)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    need = max(1, int(max((-(-int(L) // bs) for L in lens), default=1)))
    mbs = mbs or need
    if num_blocks is None:
        num_blocks = max(1, len(lens) * mbs)
    params = pa.make_params(num_seqs=len(lens), num_heads=H, num_kv_heads=Hkv, head_size=d, block_size=bs,
                            num_blocks=num_blocks, max_blocks_per_seq=mbs, dtype=dtype, scale=0.1,
                            common_prefix_len=prefix, kv_split_tokens=split, causal=causal)
    plan = pa.pa_plan_create(params, qsl, lens, block_table, device=-1)
    return plan, pa.pa_plan_get_info(plan)


def check_against_oracle(qlens, lens, **kw):
    plan, info = host_plan(qlens, lens, **kw)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    md = oracle.metadata(qsl, lens, kw.get("prefix", 0), kw.get("block_table"), kw.get("bs", 16))
    assert np.array_equal(pa.pa_plan_get_array(plan, pa.PA_ARRAY_ORDER), md["order"])
    assert np.array_equal(pa.pa_plan_get_array(plan, pa.PA_ARRAY_IS_DECODE), md["is_decode"].astype(np.int32))
    for k in ("num_decodes", "num_decode_tokens", "num_prefills", "num_prefill_tokens", "num_tokens"):
        assert info[k] == md[k], k
    assert np.array_equal(pa.pa_plan_get_array(plan, pa.PA_ARRAY_PREFIX_BLOCKS), md["prefix_blocks"])
    return plan, info


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6])
def test_config_metadata_is_bit_exact(cfg):
    qlens, lens, sp = config_lengths(cfg)
    H, Hkv, d, bs = {1: (4, 2, 64, 16), 2: (32, 8, 128, 16), 3: (32, 8, 128, 16), 4: (64, 8, 128, 64),
                     5: (32, 8, 128, 16), 6: (32, 8, 128, 16)}[cfg]
    check_against_oracle(qlens, lens, H=H, Hkv=Hkv, d=d, bs=bs)


@pytest.mark.parametrize("seed", range(6))
def test_shuffled_batches_order_decode_first(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    qlens = np.where(rng.random(B) < 0.5, 1, rng.integers(2, 300, size=B))
    lens = qlens + rng.integers(0, 2000, size=B)
    plan, info = check_against_oracle(qlens, lens)
    order = pa.pa_plan_get_array(plan, pa.PA_ARRAY_ORDER)
    nd = info["num_decodes"]
    assert np.all(qlens[order[:nd]] == 1) and np.all(qlens[order[nd:]] > 1)


def test_empty_batch():
    plan, info = host_plan([], [])
    assert info["num_tokens"] == 0 and info["num_decode_items"] == 0 and pa.pa_plan_workspace_bytes(plan) == 0


def test_split_items_cover_each_decode_exactly():
    lens = [1, 31, 32, 33, 1000, 4096]
    for split in (32, 64, 96, 1024):
        plan, info = host_plan([1] * len(lens), lens, split=split)
        assert info["kv_split_tokens"] == split
        assert info["decode_tokens_read"] == sum(lens) * 2  # every key once per KV head (Hkv = 2)
        parts = pa.pa_plan_get_array(plan, pa.PA_ARRAY_ROW_PARTIALS)
        want = [(-(-L // split)) for L in lens]
        assert list(parts) == [n if n > 1 else 0 for n in want]


def test_wide_prefill_takes_eight_waves_beside_decodes():
    """bf16 pool, head size 128, g = 4: a prefill alone runs 4-wave workgroups
    of 8 column tiles (32 positions of 4 heads); beside decodes, 8-wave
    workgroups of 16 tiles (64 positions), which fill a CU each, with or
    without a shared prefix; an e4m3 pool and fp32 queries keep 4 waves."""
    _, alone = host_plan([100], [100])
    _, mixed = host_plan([1, 100], [300, 100])
    assert alone["prefill_rows_per_item"] == 32 and mixed["prefill_rows_per_item"] == 64
    bt = np.zeros((2, 20), dtype=np.int32)
    bt[1, 1:] = np.arange(1, 20)
    # a shared prefix with decodes alone runs in the decode's launch (8-wave
    # workgroups) when the decode's workgroups have 8 waves (8 KV heads); with
    # 2 KV heads before the decode (4 waves); with prefills, the prefix pass
    # and the prefills run on the side stream beside the decode (8 waves)
    _, casc = host_plan([1, 1], [300, 200], prefix=16, block_table=bt, mbs=20, num_blocks=40, H=32, Hkv=8)
    assert casc["prefill_rows_per_item"] == 64 and casc["prefix_beside_decode"] == 1
    _, c2 = host_plan([1, 1], [300, 200], prefix=16, block_table=bt, mbs=20, num_blocks=40)
    assert c2["prefill_rows_per_item"] == 32 and c2["prefix_beside_decode"] == 0
    _, cpre = host_plan([1, 20], [300, 200], prefix=16, block_table=bt, mbs=20, num_blocks=40, H=32, Hkv=8)
    assert cpre["prefill_rows_per_item"] == 64 and cpre["prefix_beside_decode"] == 0
    _, f32 = host_plan([1, 100], [300, 100], dtype="fp32")
    assert f32["prefill_rows_per_item"] == 32
    params = pa.make_params(num_seqs=2, num_heads=8, num_kv_heads=2, head_size=128, block_size=16, num_blocks=40,
                            max_blocks_per_seq=20, dtype="bf16", scale=0.1, kv_dtype="fp8_e4m3")
    plan = pa.pa_plan_create(params, np.array([0, 1, 101], np.int32), np.array([300, 100], np.int32), device=-1)
    assert pa.pa_plan_get_info(plan)["prefill_rows_per_item"] == 32
    # g = 8: 8 heads x 32 positions beside decodes, 4 heads x 32 positions alone
    _, m8 = host_plan([1, 100], [300, 100], H=16, Hkv=2)
    _, a8 = host_plan([100], [100], H=16, Hkv=2)
    assert m8["prefill_rows_per_item"] == 32 and m8["prefill_head_groups"] == 1
    assert a8["prefill_rows_per_item"] == 32 and a8["prefill_head_groups"] == 2


def test_prefill_reads_follow_the_causal_staircase():
    # one 100-token prompt, g = 4: the work item for positions [i0, i0 + Q) reads
    # keys 0 .. i0 + Q - 1 (capped at 100), where Q is the item's position count.
    plan, info = host_plan([100], [100], H=8, Hkv=2)
    Q = info["prefill_rows_per_item"]
    assert Q in (32, 64) and info["prefill_head_groups"] == 1
    starts = range(0, 100, Q)
    assert info["num_prefill_items"] == len(starts)
    assert info["prefill_tokens_read"] == sum(min(100, i0 + Q) for i0 in starts) * 2
    # fp32 and head size 64 use 8 column tiles (32 positions for g = 4)
    plan, info = host_plan([100], [100], H=8, Hkv=2, dtype="fp32")
    assert info["num_prefill_items"] == 4
    assert info["prefill_tokens_read"] == (32 + 64 + 96 + 100) * 2
    plan, info = host_plan([100], [100], H=8, Hkv=2, d=64)
    assert info["num_prefill_items"] == 4


def test_cascade_read_counts_match_the_read_model():
    """«El especialista del plato estrella», §Qué aporta FlashInfer: the naive schedule
    reads the prefix once per request, cascade once.  With R = 50 decodes and a
    1024-token prefix: naive reads R*P + sum(s) key rows per KV head; the cascade
    schedule reads the prefix once per column group (prefill_rows_per_item query
    rows) plus the suffixes."""
    R, P, bs, Hkv = 50, 1024, 16, 2
    rng = np.random.default_rng(7)
    s = rng.integers(1, 300, size=R)
    lens = P + s
    mbs = int(max(-(-L // bs) for L in lens))
    nb = P // bs + int(sum(-(-int(x) // bs) for x in s)) + 1
    bt = np.zeros((R, mbs), dtype=np.int32)
    nxt = P // bs
    for b in range(R):
        bt[b, :P // bs] = np.arange(P // bs)
        own = -(-int(lens[b]) // bs) - P // bs
        bt[b, P // bs:P // bs + own] = np.arange(nxt, nxt + own)
        nxt += own
    model = oracle.cascade_prefix_reads(R, P, s)
    plain, _ = host_plan([1] * R, lens, Hkv=Hkv, block_table=bt, num_blocks=nb, mbs=mbs, split=8192)
    casc, _ = host_plan([1] * R, lens, Hkv=Hkv, block_table=bt, num_blocks=nb, mbs=mbs, prefix=P, split=8192)
    ip, ic = pa.pa_plan_get_info(plain), pa.pa_plan_get_info(casc)
    casc_info = ic
    assert ip["kv_tokens_read"] == model["naive"] * Hkv
    groups = -(-R // casc_info["prefill_rows_per_item"])
    # the prefix rows the plan reads, each once per KV head (the page's model),
    # and the reads of its column groups, which run together on one XCD
    assert ic["prefix_tokens_unique"] == model["prefix_cascade"] * Hkv
    assert ic["prefix_tokens_read"] == groups * P * Hkv
    assert ic["decode_tokens_read"] == int(s.sum()) * Hkv
    assert ic["kv_tokens_read"] == (groups * P + int(s.sum())) * Hkv
    assert ic["num_prefix_blocks"] == P // bs
    assert np.array_equal(pa.pa_plan_get_array(casc, pa.PA_ARRAY_PREFIX_BLOCKS), np.arange(P // bs))
    # every decode row merges the prefix parts and its suffix part
    assert np.all(pa.pa_plan_get_array(casc, pa.PA_ARRAY_ROW_PARTIALS) == P // 1024 + 1)


def _status(fn):
    with pytest.raises(pa.PagedAttnError) as ei:
        fn()
    return ei.value.status


def test_validation_errors():
    INV, UNS = pa.PA_ERR_INVALID_ARG, pa.PA_ERR_UNSUPPORTED
    # «FlashAttention y FlashInfer», §Límites y fallos: block size must be a multiple of 16
    assert _status(lambda: host_plan([1], [10], bs=24)) == INV
    assert _status(lambda: host_plan([1], [10], bs=8)) == INV
    # «AttentionBackend: capa de abstracción», §Límites y fallos: head size / dtype limits
    assert _status(lambda: host_plan([1], [10], d=96)) == UNS
    assert _status(lambda: host_plan([1], [10], d=256)) == UNS
    assert _status(lambda: host_plan([1], [10], dtype=7)) == UNS
    assert _status(lambda: host_plan([1], [10], H=6, Hkv=4)) == INV
    assert _status(lambda: host_plan([1, 0], [10, 4])) == INV           # a sequence without queries
    assert _status(lambda: host_plan([5], [3])) == INV                   # seq_len < query tokens
    assert _status(lambda: host_plan([1], [40], mbs=2)) == INV           # block table row too short
    assert _status(lambda: host_plan([1], [10], split=48)) == INV        # split not a multiple of 32
    bt = np.array([[0, 1, 7]], dtype=np.int32)
    assert _status(lambda: host_plan([1], [40], block_table=bt, num_blocks=5)) == INV  # id outside the pool
    # cascade preconditions
    bt2 = np.array([[0, 1, 2], [0, 1, 3]], dtype=np.int32)
    assert _status(lambda: host_plan([1, 1], [40, 45], prefix=32)) == INV                       # no table
    assert _status(lambda: host_plan([1, 1], [40, 45], block_table=bt2, num_blocks=4, prefix=24)) == INV
    assert _status(lambda: host_plan([1, 1], [40, 45], block_table=bt2, num_blocks=4, prefix=48)) == INV
    assert _status(lambda: host_plan([1, 9], [40, 40], block_table=bt2, num_blocks=4, prefix=48)) == INV
    ok, _ = host_plan([1, 1], [40, 45], block_table=bt2, num_blocks=4, prefix=32)
    assert pa.pa_plan_get_info(ok)["common_prefix_len"] == 32


def test_query_start_loc_must_start_at_zero():
    params = pa.make_params(num_seqs=1, num_heads=2, num_kv_heads=1, head_size=64, block_size=16, num_blocks=4,
                            max_blocks_per_seq=4, dtype="bf16", scale=0.1)
    assert _status(lambda: pa.pa_plan_create(params, [1, 2], [5], None, device=-1)) == pa.PA_ERR_INVALID_ARG


def test_host_only_plan_cannot_run():
    plan, _ = host_plan([1], [10])
    assert _status(lambda: pa.pa_forward(plan, 16, 16, 16, None, None, 16, None, None, 0, stream=0)) == pa.PA_ERR_INVALID_ARG


def test_workspace_size_accounts_for_partials():
    plan, info = host_plan([1, 1], [100, 1000], split=64, H=8)
    n = info["num_partials"]
    assert n == 2 + 16
    ws = pa.pa_plan_workspace_bytes(plan)
    assert ws >= n * 8 * 128 * 4 + n * 8 * 4


def _list_budgets(info, n):
    """Budget of each of n balanced lists: W, or W - W/128 (even list) and
    W + W/128 (odd list) when the plan sizes them by XCD."""
    W = info["decode_list_tokens"]
    if not info["decode_list_xcd_budgets"]:
        return np.full(n, W)
    return np.array([W - W // 128 if i % 2 == 0 else W + W // 128 for i in range(n)])


def _decode_schedule(plan, info):
    lists = pa.pa_plan_get_array(plan, pa.PA_ARRAY_DECODE_LISTS)
    spans = pa.pa_plan_get_array(plan, pa.PA_ARRAY_DECODE_SPANS).reshape(-1, 3)
    assert len(lists) == info["num_decode_lists"] + 1 and len(spans) == info["num_decode_items"]
    assert lists[0] == 0 and lists[-1] == len(spans) and np.all(np.diff(lists) >= 1)
    return lists, spans


@pytest.mark.parametrize("seed", range(4))
def test_balanced_decode_lists_partition_the_keys(seed):
    """A batch of decodes alone, automatic split: the lists cut the decode keys,
    sequence after sequence in decode-first order, into runs of equal cost
    (keys, plus decode_item_keys for each item); every key of every sequence
    is covered exactly once, in order."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 60))
    lens = rng.integers(1, 9000, size=B)
    plan, info = host_plan([1] * B, lens, H=32, Hkv=8)
    lists, spans = _decode_schedule(plan, info)
    W, ik = info["decode_list_tokens"], info["decode_item_keys"]
    assert W > 0 and info["kv_split_tokens"] == W and ik > 0
    # decodes alone, one workgroup per list: the measured item cost and the
    # XCD budgets
    assert ik == 16 and info["decode_list_xcd_budgets"] == 1
    sizes = np.array([int((spans[a:b, 2] - spans[a:b, 1]).sum()) for a, b in zip(lists[:-1], lists[1:])])
    cost = sizes + ik * np.diff(lists)
    bud = _list_budgets(info, len(sizes))
    assert np.all(cost[:-1] > bud[:-1] - 32 - ik) and np.all(cost <= bud) and sizes[-1] > 0
    # items start on 32-key boundaries of their sequence (16-key tiles never
    # straddle a physical block)
    assert np.all(spans[:, 1] % 32 == 0)
    assert info["num_decode_lists"] <= 256  # one list per resident group of waves (host plans: 256 CUs)
    order = pa.pa_plan_get_array(plan, pa.PA_ARRAY_ORDER)
    pos = 0
    for b in order:  # all decodes: the spans walk the sequences in order
        k = 0
        while k < lens[b]:
            seq, k0, k1 = spans[pos]
            assert seq == b and k0 == k and k1 > k0
            k = k1
            pos += 1
    assert pos == len(spans)
    parts = np.bincount(spans[:, 0], minlength=B)
    assert np.array_equal(pa.pa_plan_get_array(plan, pa.PA_ARRAY_ROW_PARTIALS), np.where(parts > 1, parts, 0))
    assert info["decode_tokens_read"] == int(lens.sum()) * 8


def _lists_needed(lens, W, ik, xcd):
    """The list cut of the balanced decode schedule, counted: a list closes
    when less than 32 of its budget (W, or W -+ W/128 for even / odd lists
    with XCD budgets) is left, or before an item (which costs ik) that would
    start with less."""
    def bud(i):
        return W if not xcd else (W - W // 128 if i % 2 == 0 else W + W // 128)
    n, filled = 0, 0
    for L in lens:
        k0 = 0
        while k0 < L:
            if bud(n) - filled - ik < 32:
                n, filled = n + 1, 0
            filled += ik
            room = bud(n) - filled
            take = L - k0 if L - k0 <= room else room // 32 * 32
            k0 += take
            filled += take
            if bud(n) - filled < 32:
                n, filled = n + 1, 0
    return n + (1 if filled > 0 else 0)


def test_balanced_decode_lists_never_exceed_the_resident_groups():
    """Each list may close with up to 31 keys of its budget unused (cuts inside
    a sequence fall on 32-key boundaries), or 31 + decode_item_keys before an
    item; the planner sizes the lists so that the keys still fit in one list
    per resident group of waves (host plans: 256 CUs, one 8-wave workgroup per
    CU at Hkv = 8), never spilling into a second round, and takes the smallest
    budget that does (one budget step less would need more lists).  The
    suffix lengths of the cascade batch (128 decodes, U[256, 2048]) once gave
    258 lists."""
    from workloads import config_lengths
    _, L, sp = config_lengths(5)
    suffix = [int(x) - 16 * sp for x in L]
    cases = [suffix] + [list(np.random.default_rng(500 + s).integers(1, 4096, size=int(n)))
                        for s, n in enumerate([37, 128, 255, 256, 257, 400, 1000])]
    for lens in cases:
        plan, info = host_plan([1] * len(lens), lens, H=32, Hkv=8)
        lists, spans = _decode_schedule(plan, info)
        need = -(-int(np.sum(lens)) // 256)
        assert info["num_decode_lists"] <= min(256, need), (len(lens), info["num_decode_lists"])
        W, ik = info["decode_list_tokens"], info["decode_item_keys"]
        sizes = np.array([int((spans[a:b, 2] - spans[a:b, 1]).sum()) for a, b in zip(lists[:-1], lists[1:])])
        cost = sizes + ik * np.diff(lists)
        bud = _list_budgets(info, len(sizes))
        assert sizes.sum() == int(np.sum(lens)) and np.all(cost <= bud) and np.all(cost[:-1] > bud[:-1] - 32 - ik)
        # the cut the test counts is the planner's, and the budget is the
        # smallest: the same cut with W - 1 needs more lists
        xcd = info["decode_list_xcd_budgets"]
        assert _lists_needed(lens, W, ik, xcd) == info["num_decode_lists"]
        if W - 1 >= 64 + ik:
            assert _lists_needed(lens, W - 1, ik, xcd) > min(256, need)


def test_decode_lists_are_single_items_with_an_explicit_split():
    lens = [100, 5000, 40, 700]
    plan, info = host_plan([1, 1, 1, 1], lens, split=64)
    lists, spans = _decode_schedule(plan, info)
    assert np.array_equal(lists, np.arange(len(spans) + 1)) and info["decode_list_tokens"] == 0


def test_balanced_decode_lists_start_past_a_shared_prefix():
    """With a shared prefix the balanced lists cut only the keys past it; each
    decode row merges its prefix chunks with its suffix pieces."""
    P = 32
    lens = [100, 5000, 40, 700]
    bt = np.arange(4 * 313, dtype=np.int32).reshape(4, 313)
    bt[:, :P // 16] = bt[0, :P // 16]
    plan, info = host_plan([1, 1, 1, 1], lens, prefix=P, block_table=bt, mbs=313, H=32, Hkv=8)
    lists, spans = _decode_schedule(plan, info)
    assert info["decode_list_tokens"] > 0 and info["num_decode_lists"] <= 256
    # beside a shared-prefix pass: one budget for all lists, items at 24 keys
    # when the pass shares the decode's launch (64 otherwise)
    assert info["decode_item_keys"] == (24 if info["prefix_beside_decode"] else 64)
    assert info["decode_list_xcd_budgets"] == 0
    assert np.all(spans[:, 1] >= P) and np.all(spans[:, 1] % 32 == 0)
    assert info["decode_tokens_read"] == sum(L - P for L in lens) * 8
    order = pa.pa_plan_get_array(plan, pa.PA_ARRAY_ORDER)
    pos = 0
    for b in order:  # the spans walk each sequence's suffix in order
        k = P
        while k < lens[b]:
            seq, k0, k1 = spans[pos]
            assert seq == b and k0 == k and k1 > k0
            k = k1
            pos += 1
    assert pos == len(spans)
    parts = np.bincount(spans[:, 0], minlength=4)
    n_pc = info["num_prefix_items"] // max(1, -(-4 // info["prefill_rows_per_item"]))
    assert np.array_equal(pa.pa_plan_get_array(plan, pa.PA_ARRAY_ROW_PARTIALS), parts + n_pc)


def _covers_decodes_in_order(plan, lens, spans):
    order = pa.pa_plan_get_array(plan, pa.PA_ARRAY_ORDER)
    pos = 0
    for b in order:
        k = 0
        while pos < len(spans) and spans[pos][0] == b:
            assert spans[pos][1] == k and spans[pos][2] > k
            k = spans[pos][2]
            pos += 1
        if k:
            assert k == lens[b]
    assert pos == len(spans)


@pytest.mark.parametrize("heavy", ["decode", "prefill"])
def test_decode_lists_beside_prefills_take_a_share_of_the_machine(heavy):
    """Beside prefills the balanced lists take between a quarter and three
    quarters of the resident wave groups (host plans: 256 CUs, one workgroup
    of two waves per list at H=8, Hkv=2): close to three quarters when the
    decodes dominate, fewer when the prefill does; the keys are still covered
    once, in order."""
    if heavy == "decode":
        qlens, lens = [1] * 64 + [32], [8000] * 64 + [32]
    else:
        qlens, lens = [1] * 40 + [4096], [3000] * 40 + [4096]
    plan, info = host_plan(qlens, lens)
    lists, spans = _decode_schedule(plan, info)
    n = info["num_decode_lists"]
    assert info["decode_list_tokens"] > 0 and 64 <= n <= 192
    # beside prefills: one budget for all lists, items at 64 keys
    assert info["decode_item_keys"] == 64 and info["decode_list_xcd_budgets"] == 0
    if heavy == "decode":
        assert n >= 180
    else:
        assert n <= 128
    _covers_decodes_in_order(plan, np.asarray(lens), spans[:, :3])


def test_prefix_beside_decode_takes_cus_of_its_own():
    """Shared prefix, decodes alone (the cascade workload's shape): the prefix
    pass is cut into chunks whose 8-wave units (chunk, 64-row column group, KV
    head) each take one CU, and the decode lists cover the other CUs; the
    chunks tile [0, P) and every row merges the prefix chunks with its suffix
    pieces."""
    qlens, lens, sp = config_lengths(5)
    R, P, bs, Hkv = len(lens), 16384, 16, 8
    mbs = int(max(-(-int(L) // bs) for L in lens))
    bt = np.zeros((R, mbs), dtype=np.int32)
    nxt = P // bs
    for b in range(R):
        bt[b, :P // bs] = np.arange(P // bs)
        own = -(-int(lens[b]) // bs) - P // bs
        bt[b, P // bs:P // bs + own] = np.arange(nxt, nxt + own)
        nxt += own
    plan, info = host_plan(qlens, lens, H=32, Hkv=Hkv, bs=bs, block_table=bt, num_blocks=nxt, mbs=mbs, prefix=P)
    assert info["prefix_beside_decode"] == 1 and info["prefill_rows_per_item"] == 64
    groups = -(-R // 64)
    units = info["num_prefix_items"] * Hkv
    chunks = info["num_prefix_items"] // groups
    assert info["num_prefix_items"] == chunks * groups and 1 <= chunks <= P // 64
    assert 8 <= units <= 256 - 8
    # decode lists: one 8-wave group per CU the prefix leaves free (host-only
    # plans assume 256 CUs and one decode workgroup per CU)
    assert info["num_decode_lists"] <= 256 - units
    assert info["prefix_tokens_read"] == groups * P * Hkv and info["prefix_tokens_unique"] == P * Hkv
    parts = pa.pa_plan_get_array(plan, pa.PA_ARRAY_ROW_PARTIALS)
    spans = pa.pa_plan_get_array(plan, pa.PA_ARRAY_DECODE_SPANS).reshape(-1, 3)
    pieces = np.bincount(spans[:, 0], minlength=R)
    assert np.all(spans[:, 1] >= P)
    assert np.array_equal(parts, chunks + pieces)


def test_prefix_pass_covers_decode_rows_only():
    """With a shared prefix, prefill rows attend to their whole context in
    their own items (one contribution, no partial record); the prefix pass
    covers the decode rows, one run of consecutive rows at a time, and each
    decode row merges its prefix chunks with its suffix pieces."""
    P, bs = 64, 16
    qlens = np.array([1, 1, 30, 1, 20, 1, 1])       # decode runs: rows [0, 2), [32, 33), [53, 55)
    lens = np.array([P + 40, P + 300, P + 50, P + 7, P + 100, P + 1, P + 64])
    mbs = int(max(-(-int(L) // bs) for L in lens))
    bt = np.zeros((len(lens), mbs), dtype=np.int32)
    nxt = P // bs
    for b in range(len(lens)):
        bt[b, :P // bs] = np.arange(P // bs)
        own = -(-int(lens[b]) // bs) - P // bs
        bt[b, P // bs:P // bs + own] = np.arange(nxt, nxt + own)
        nxt += own
    plan, info = host_plan(qlens, lens, H=8, Hkv=2, block_table=bt, num_blocks=nxt, mbs=mbs, prefix=P)
    qsl = np.concatenate([[0], np.cumsum(qlens)])
    parts = pa.pa_plan_get_array(plan, pa.PA_ARRAY_ROW_PARTIALS)
    pre_rows = np.concatenate([np.arange(qsl[b], qsl[b + 1]) for b in range(len(lens)) if qlens[b] > 1])
    dec_rows = qsl[:-1][qlens == 1]
    assert np.all(parts[pre_rows] == 0)
    assert np.all(parts[dec_rows] >= 2)                 # at least one prefix chunk and one suffix piece
    Q = info["prefill_rows_per_item"]
    runs = [(0, 2), (32, 33), (53, 55)]
    items_per_chunk = sum(-(-(e - s) // Q) for s, e in runs)
    assert info["num_prefix_items"] % items_per_chunk == 0
    # every row group of every run reads the whole prefix once per KV head (2)
    assert info["prefix_tokens_read"] == items_per_chunk * P * info["prefill_head_groups"] * 2
    # prefill items read their whole context, prefix included
    pre_keys = sum(sum(min(int(lens[b]), int(lens[b]) - int(qlens[b]) + i0 + min(Q, int(qlens[b]) - i0))
                       for i0 in range(0, int(qlens[b]), Q)) for b in range(len(lens)) if qlens[b] > 1)
    assert info["prefill_tokens_read"] == pre_keys * 2 * info["prefill_head_groups"]


@pytest.mark.parametrize("seed", range(8))
def test_cascade_schedules_cover_rows_and_fit_the_chip(seed):
    """Random batches with a shared prefix (8 KV heads, so decodes alone take
    the fused launch): the prefix chunks tile [0, P); with decodes alone, the
    prefix units (chunks x 64-row groups x KV heads) and the decode lists fit
    the 256 CUs a host-only plan assumes; every decode row merges its prefix
    chunks with its suffix pieces, and prefill rows have no partial record."""
    rng = np.random.default_rng(100 + seed)
    bs = 16
    P = bs * int(rng.integers(1, 300))
    B = int(rng.integers(1, 200))
    prefills = seed % 2 == 1
    qlens = np.where(rng.random(B) < (0.1 if prefills else 0.0), rng.integers(2, 300, size=B), 1)
    lens = P + qlens - 1 + rng.integers(1, 3000, size=B)
    mbs = int(max(-(-int(L) // bs) for L in lens))
    bt = np.zeros((B, mbs), dtype=np.int32)
    nxt = P // bs
    for b in range(B):
        bt[b, :P // bs] = np.arange(P // bs)
        own = -(-int(lens[b]) // bs) - P // bs
        bt[b, P // bs:P // bs + own] = np.arange(nxt, nxt + own)
        nxt += own
    plan, info = host_plan(qlens, lens, H=32, Hkv=8, bs=bs, block_table=bt, num_blocks=nxt, mbs=mbs, prefix=P)
    qsl = np.concatenate([[0], np.cumsum(qlens)])
    dec = qlens == 1
    parts = pa.pa_plan_get_array(plan, pa.PA_ARRAY_ROW_PARTIALS)
    spans = pa.pa_plan_get_array(plan, pa.PA_ARRAY_DECODE_SPANS).reshape(-1, 3)
    pieces = np.bincount(spans[:, 0], minlength=B)
    assert np.all(spans[:, 1] >= P)
    assert info["prefix_beside_decode"] == (0 if prefills and (~dec).any() else 1)
    # decode rows: consecutive runs of decode rows, grouped by the prefix item row count
    Q = info["prefill_rows_per_item"]
    runs, start = [], None
    for b in range(B):
        if dec[b] and start is None:
            start = b
        if (not dec[b] or b == B - 1) and start is not None:
            end = b + 1 if dec[b] else b
            runs.append(end - start)
            start = None
    groups = sum(-(-n // Q) for n in runs)
    assert info["num_prefix_items"] % groups == 0
    chunks = info["num_prefix_items"] // groups
    assert 1 <= chunks <= -(-P // 64)
    assert info["prefix_tokens_read"] == groups * P * info["prefill_head_groups"] * 8
    rows_dec = qsl[:-1][dec]
    want = np.where(chunks + pieces[dec] > 1, chunks + pieces[dec], 0)
    assert np.array_equal(parts[rows_dec], want)
    if (~dec).any():
        pre_rows = np.concatenate([np.arange(qsl[b], qsl[b + 1]) for b in range(B) if not dec[b]])
        assert np.all(parts[pre_rows] == 0)
    if info["prefix_beside_decode"]:
        units = info["num_prefix_items"] * 8 * info["prefill_head_groups"]
        assert units + info["num_decode_lists"] <= 256


def test_decode_share_beside_prefills_follows_the_pool_type():
    """The chunked-prefill mixed batch (192 decodes, four 512-token chunks):
    the decode lists take the share the two parts' estimated times give,
    capped at three quarters for bf16 (192 of 256 groups); over an e4m3 pool
    the prefill's slower rate (0.7 against 0.9 PFLOP/s) and the decode's
    halved bytes leave the decode about 60 % (153 lists)."""
    from workloads import config_lengths
    q, L, _ = config_lengths(4)
    qsl = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
    mbs = int(-(-int(L.max()) // 64))
    counts = {}
    for kvd in ("same", "fp8_e4m3"):
        p = pa.make_params(num_seqs=len(L), num_heads=64, num_kv_heads=8, head_size=128, block_size=64,
                           num_blocks=len(L) * mbs, max_blocks_per_seq=mbs, dtype="bf16", scale=128 ** -0.5,
                           kv_dtype=kvd)
        info = pa.pa_plan_get_info(pa.pa_plan_create(p, qsl, L.astype(np.int32), None, device=-1))
        assert info["num_prefills"] == 4 and info["decode_item_keys"] == 64
        counts[kvd] = info["num_decode_lists"]
    assert counts == {"same": 192, "fp8_e4m3": 153}
