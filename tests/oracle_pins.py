"""Pins for the CPU oracle: each check ties it to something other than itself.

Every ``check_*`` takes the oracle module as its argument and raises on a
mismatch.  ``test_oracle_pins.py`` runs them against the real oracle;
``test_oracle_mutations.py`` runs them against deliberately broken copies of it
to show that a plausible mistake anywhere in the oracle fails at least one pin.

The logical-to-physical writer ``pool_from_logical`` below places contiguous K/V
into pages by reshaping whole blocks, a different mechanism from the oracle's
index arithmetic, so the round trip through ``gather`` is a real check.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pool_from_logical(Ks, Vs, block_size, *, seed=0, spare=3, shared_prefix_blocks=0):
    """Write per-sequence contiguous K/V ``[L_b, Hkv, d]`` into a randomly placed pool.

    Whole blocks are written by reshaping ``[n_pages * bs, Hkv, d]`` into
    ``[n_pages, bs, Hkv, d]``; unused pages and past-the-end slots are NaN.  With
    ``shared_prefix_blocks`` the first blocks of every sequence are the same
    physical pages (taken from sequence 0's values).
    """
    bs = block_size
    Hkv, d = Ks[0].shape[1:]
    pages = [-(-len(K) // bs) for K in Ks]
    sp = shared_prefix_blocks
    total = sp + sum(p - sp for p in pages)
    nb = total + spare
    perm = np.random.default_rng(seed).permutation(nb)
    pool = np.full((nb, 2, bs, Hkv, d), np.nan, dtype=np.float32)
    bt = np.full((len(Ks), max(pages)), perm[-1], dtype=np.int32)

    def write(ids, K, V, n):
        padK = np.full((n * bs, Hkv, d), np.nan, dtype=np.float32)
        padV = padK.copy()
        padK[:len(K)] = K
        padV[:len(V)] = V
        pool[ids, 0] = padK.reshape(n, bs, Hkv, d)
        pool[ids, 1] = padV.reshape(n, bs, Hkv, d)

    prefix_ids = perm[:sp]
    if sp:
        write(prefix_ids, Ks[0][:sp * bs], Vs[0][:sp * bs], sp)
    cur = sp
    for b, (K, V) in enumerate(zip(Ks, Vs)):
        n = pages[b] - sp
        ids = perm[cur:cur + n]
        cur += n
        write(ids, K[sp * bs:], V[sp * bs:], n)
        bt[b, :sp] = prefix_ids
        bt[b, sp:pages[b]] = ids
    return pool, bt


def _qsl(qlens):
    return np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)


def _random_logical(lens, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    Ks = [rng.standard_normal((L, Hkv, d)).astype(np.float32) for L in lens]
    Vs = [rng.standard_normal((L, Hkv, d)).astype(np.float32) for L in lens]
    return Ks, Vs


# A small mixed batch: two decodes, a chunk with context, a full prefill, a chunk.
MIX_Q = [1, 1, 16, 37, 5]
MIX_L = [17, 33, 64, 37, 40]


# ---------------------------------------------------------------------------

def check_kv_cache_shape(O):
    g = _golden("kv_cache_shape.json")
    for case in g["cases"]:
        assert tuple(O.kv_cache_shape(*case["args"])) == tuple(case["shape"])
    for bs in g["rejected_block_sizes"]:
        try:
            O.kv_cache_shape(4, bs, 2, 64)
        except ValueError:
            continue
        raise AssertionError(f"block size {bs} accepted")


def check_gather_roundtrip(O):
    for bs, lens in ((16, [1, 15, 16, 17, 50]), (32, [33, 64, 5]), (48, [100, 47])):
        Ks, Vs = _random_logical(lens, 3, 8, seed=bs)
        pool, bt = pool_from_logical(Ks, Vs, bs, seed=bs + 1)
        for b, L in enumerate(lens):
            K, V = O.gather(pool, bt[b], L)
            assert K.shape == (L, 3, 8)
            assert np.array_equal(K, Ks[b]) and np.array_equal(V, Vs[b])


def check_single_key(O):
    # One key per sequence; the other slots of the page are NaN.  The output is
    # that key's V row exactly and the LSE is the single scaled score.
    Ks, Vs = _random_logical([1, 1], 2, 32, seed=3)
    pool, bt = pool_from_logical(Ks, Vs, 16, seed=4)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 32)).astype(np.float32)
    scale = 0.37
    out, lse = O.attention(q, pool, bt, _qsl([1, 1]), np.array([1, 1]), scale, dtype="fp32")
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], Vs[b][0, h // 2].astype(np.float64))
            s = scale * math.fsum(float(a) * float(c) for a, c in zip(q[b, h], Ks[b][0, h // 2]))
            assert abs(lse[b, h] - s) < 1e-12


def check_equal_scores(O):
    # q = 0: every visible score is 0, so the output is the plain mean of the
    # visible V rows and the LSE is ln(number of visible keys).
    H, Hkv, d = 6, 2, 8
    g = H // Hkv
    Ks, Vs = _random_logical(MIX_L, Hkv, d, seed=6)
    pool, bt = pool_from_logical(Ks, Vs, 16, seed=7)
    q = np.zeros((sum(MIX_Q), H, d), dtype=np.float32)
    qsl = _qsl(MIX_Q)
    for causal in (True, False):
        out, lse = O.attention(q, pool, bt, qsl, np.array(MIX_L), 0.5, dtype="fp32", causal=causal)
        for b, (qb, L) in enumerate(zip(MIX_Q, MIX_L)):
            c = L - qb
            for i in range(qb):
                n = (c + i + 1) if causal else L
                r = qsl[b] + i
                for h in range(H):
                    exp_o = Vs[b][:n, h // g].astype(np.float64).mean(axis=0)
                    assert np.max(np.abs(out[r, h] - exp_o)) < 1e-12
                    assert abs(lse[r, h] - math.log(n)) < 1e-12


def check_ramp_needle(O):
    # K[t, :, 0] = 256 t, q[., 0] = 1: the score grows by 256*scale = 64 per key,
    # so all weight sits on the last visible key (next one down: e^-64).
    H, Hkv, d, scale = 4, 2, 16, 0.25
    g = H // Hkv
    Ks, Vs = [], []
    for L in MIX_L:
        K = np.zeros((L, Hkv, d), dtype=np.float32)
        K[:, :, 0] = 256.0 * np.arange(L)[:, None]
        V = (np.arange(L)[:, None, None] + 1000.0 * np.arange(Hkv)[None, :, None]
             + 0.001 * np.arange(d)[None, None, :]).astype(np.float32)
        Ks.append(K)
        Vs.append(V)
    pool, bt = pool_from_logical(Ks, Vs, 16, seed=8)
    q = np.zeros((sum(MIX_Q), H, d), dtype=np.float32)
    q[:, :, 0] = 1.0
    qsl = _qsl(MIX_Q)
    out, lse = O.attention(q, pool, bt, qsl, np.array(MIX_L), scale, dtype="fp32")
    for b, (qb, L) in enumerate(zip(MIX_Q, MIX_L)):
        c = L - qb
        for i in range(qb):
            r = qsl[b] + i
            for h in range(H):
                assert np.max(np.abs(out[r, h] - Vs[b][c + i, h // g])) < 1e-9
                assert abs(lse[r, h] - 64.0 * (c + i)) < 1e-9


def check_bruteforce_tiny(O):
    # Pure-Python loops with math.fsum / math.exp, indexing the pool directly.
    H, Hkv, d, bs, scale = 4, 2, 8, 16, 0.3
    g = H // Hkv
    lens, qlens = [17, 33, 40, 20], [1, 1, 8, 20]
    Ks, Vs = _random_logical(lens, Hkv, d, seed=9)
    pool, bt = pool_from_logical(Ks, Vs, bs, seed=10)
    rng = np.random.default_rng(11)
    q = rng.standard_normal((sum(qlens), H, d)).astype(np.float32)
    qsl = _qsl(qlens)
    out, lse = O.attention(q, pool, bt, qsl, np.array(lens), scale, dtype="fp32")
    for b in range(len(lens)):
        c = lens[b] - qlens[b]
        for i in range(qlens[b]):
            r = int(qsl[b]) + i
            for h in range(H):
                kv = h // g
                sc = []
                for t in range(c + i + 1):
                    blk, slot = int(bt[b][t // bs]), t % bs
                    sc.append(scale * math.fsum(float(q[r, h, j]) * float(pool[blk, 0, slot, kv, j])
                                                for j in range(d)))
                m = max(sc)
                w = [math.exp(s - m) for s in sc]
                Z = math.fsum(w)
                for j in range(d):
                    val = math.fsum(w[t] * float(pool[int(bt[b][t // bs]), 1, t % bs, kv, j])
                                    for t in range(len(w))) / Z
                    assert abs(out[r, h, j] - val) < 1e-12
                assert abs(lse[r, h] - (m + math.log(Z))) < 1e-12


def check_sdpa_special_case(O):
    # torch's CPU attention in float64 with an explicit boolean-derived additive
    # mask (key t visible iff t <= c + i) and K/V heads repeated g times.
    import torch
    H, Hkv, d, scale = 8, 2, 16, 0.2
    g = H // Hkv
    lens, qlens = [37, 64, 30, 50], [37, 64, 10, 1]
    Ks, Vs = _random_logical(lens, Hkv, d, seed=12)
    pool, bt = pool_from_logical(Ks, Vs, 16, seed=13)
    rng = np.random.default_rng(14)
    q = rng.standard_normal((sum(qlens), H, d)).astype(np.float32)
    qsl = _qsl(qlens)
    out, lse = O.attention(q, pool, bt, qsl, np.array(lens), scale, dtype="fp32")
    for b, (L, qb) in enumerate(zip(lens, qlens)):
        c = L - qb
        Q = torch.from_numpy(q[qsl[b]:qsl[b + 1]].astype(np.float64)).transpose(0, 1)[None]
        K = torch.from_numpy(np.repeat(Ks[b], g, axis=1).astype(np.float64)).transpose(0, 1)[None]
        V = torch.from_numpy(np.repeat(Vs[b], g, axis=1).astype(np.float64)).transpose(0, 1)[None]
        vis = np.arange(L)[None, :] <= (c + np.arange(qb))[:, None]
        am = torch.from_numpy(np.where(vis, 0.0, -np.inf))
        o_ref, lse_ref = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
            Q.contiguous(), K.contiguous(), V.contiguous(), 0.0, False, attn_mask=am, scale=scale)[:2]
        o_ref = o_ref[0].transpose(0, 1).numpy()
        lse_ref = lse_ref[0].transpose(0, 1).numpy()
        assert np.max(np.abs(out[qsl[b]:qsl[b + 1]] - o_ref)) < 1e-10
        assert np.max(np.abs(lse[qsl[b]:qsl[b + 1]] - lse_ref)) < 1e-10


def check_cascade_equals_full(O):
    # Two shared blocks (32 tokens) at the front of every table.
    H, Hkv, d, bs = 4, 2, 16, 16
    lens, qlens = [50, 33, 60, 90], [1, 1, 8, 3]
    rng = np.random.default_rng(15)
    prefix_K = rng.standard_normal((32, Hkv, d)).astype(np.float32)
    prefix_V = rng.standard_normal((32, Hkv, d)).astype(np.float32)
    Ks, Vs = _random_logical(lens, Hkv, d, seed=16)
    for K, V in zip(Ks, Vs):
        K[:32], V[:32] = prefix_K, prefix_V
    pool, bt = pool_from_logical(Ks, Vs, bs, seed=17, shared_prefix_blocks=2)
    q = rng.standard_normal((sum(qlens), H, d)).astype(np.float32)
    qsl = _qsl(qlens)
    full = O.attention(q, pool, bt, qsl, np.array(lens), 0.25, dtype="fp32")
    casc = O.cascade_attention(q, pool, bt, qsl, np.array(lens), 0.25, 32, dtype="fp32")
    assert np.max(np.abs(full[0] - casc[0])) < 1e-12
    assert np.max(np.abs(full[1] - casc[1])) < 1e-12
    # the prefix blocks reported by the metadata are the shared physical blocks
    md = O.metadata(qsl, np.array(lens), 32, bt, bs)
    assert list(md["prefix_blocks"]) == list(bt[0, :2])


def check_chunk_consistency(O):
    # One 90-token prompt processed whole, or as three chunks whose context is
    # everything before them: each row must come out the same.
    H, Hkv, d = 4, 1, 16
    Ks, Vs = _random_logical([90], Hkv, d, seed=18)
    pool, bt1 = pool_from_logical(Ks, Vs, 16, seed=19)
    rng = np.random.default_rng(20)
    q = rng.standard_normal((90, H, d)).astype(np.float32)
    whole = O.attention(q, pool, bt1, _qsl([90]), np.array([90]), 0.3, dtype="fp32")
    bt3 = np.repeat(bt1, 3, axis=0)
    chunks = O.attention(q, pool, bt3, _qsl([30, 34, 26]), np.array([30, 64, 90]), 0.3, dtype="fp32")
    assert np.max(np.abs(whole[0] - chunks[0])) < 1e-12
    assert np.max(np.abs(whole[1] - chunks[1])) < 1e-12


def check_gqa_expansion(O):
    # GQA with g = 4 equals MHA over a pool whose KV heads are repeated 4 times.
    H, Hkv, d = 8, 2, 16
    Ks, Vs = _random_logical(MIX_L, Hkv, d, seed=21)
    pool, bt = pool_from_logical(Ks, Vs, 16, seed=22)
    rng = np.random.default_rng(23)
    q = rng.standard_normal((sum(MIX_Q), H, d)).astype(np.float32)
    qsl = _qsl(MIX_Q)
    gqa = O.attention(q, pool, bt, qsl, np.array(MIX_L), 0.3, dtype="fp32")
    mha = O.attention(q, np.repeat(pool, H // Hkv, axis=3), bt, qsl, np.array(MIX_L), 0.3, dtype="fp32")
    assert np.max(np.abs(gqa[0] - mha[0])) < 1e-12
    assert np.max(np.abs(gqa[1] - mha[1])) < 1e-12


def check_batch_permutation(O):
    # Reordering the sequences of a batch only reorders the output rows.
    H, Hkv, d = 4, 2, 16
    Ks, Vs = _random_logical(MIX_L, Hkv, d, seed=24)
    pool, bt = pool_from_logical(Ks, Vs, 16, seed=25)
    rng = np.random.default_rng(26)
    q = rng.standard_normal((sum(MIX_Q), H, d)).astype(np.float32)
    qsl = _qsl(MIX_Q)
    ref = O.attention(q, pool, bt, qsl, np.array(MIX_L), 0.3, dtype="fp32")
    perm = [3, 0, 4, 2, 1]
    qlens2 = [MIX_Q[p] for p in perm]
    qsl2 = _qsl(qlens2)
    rows = np.concatenate([np.arange(qsl[p], qsl[p + 1]) for p in perm])
    out = O.attention(q[rows], pool, bt[perm], qsl2, np.array([MIX_L[p] for p in perm]), 0.3, dtype="fp32")
    assert np.array_equal(out[0], ref[0][rows]) and np.array_equal(out[1], ref[1][rows])
    md = O.metadata(qsl2, np.array([MIX_L[p] for p in perm]))
    is_dec = [q == 1 for q in qlens2]
    assert list(md["order"]) == [i for i in range(5) if is_dec[i]] + [i for i in range(5) if not is_dec[i]]


def check_block_permutation(O):
    # Moving pages to other physical slots and rewriting the table changes nothing.
    H, Hkv, d = 4, 2, 16
    Ks, Vs = _random_logical(MIX_L, Hkv, d, seed=27)
    pool, bt = pool_from_logical(Ks, Vs, 16, seed=28)
    rng = np.random.default_rng(29)
    q = rng.standard_normal((sum(MIX_Q), H, d)).astype(np.float32)
    qsl = _qsl(MIX_Q)
    ref = O.attention(q, pool, bt, qsl, np.array(MIX_L), 0.3, dtype="fp32")
    perm = rng.permutation(pool.shape[0])
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    out = O.attention(q, pool2, perm[bt].astype(np.int32), qsl, np.array(MIX_L), 0.3, dtype="fp32")
    assert np.array_equal(out[0], ref[0]) and np.array_equal(out[1], ref[1])


def check_metadata_golden(O):
    for case in _golden("decode_first.json")["cases"]:
        qsl = _qsl(case["query_lens"])
        md = O.metadata(qsl, np.array(case["seq_lens"]))
        assert [int(x) for x in md["is_decode"]] == case["is_decode"]
        assert [int(x) for x in md["order"]] == case["order"]
        for k in ("num_decodes", "num_decode_tokens", "num_prefills", "num_prefill_tokens"):
            assert md[k] == case[k], k
        assert [int(x) for x in md["context_lens"]] == case["context_lens"]
        assert [int(x) for x in md["is_chunked"]] == case["is_chunked"]


def check_metadata_cascade_errors(O):
    qsl = _qsl([1, 1])
    bt = np.array([[3, 4, 5], [3, 4, 6]], dtype=np.int32)
    md = O.metadata(qsl, np.array([40, 45]), 32, bt, 16)
    assert list(md["prefix_blocks"]) == [3, 4]
    bad = [
        (np.array([40, 45]), 24, bt),                                   # not whole blocks
        (np.array([40, 45]), 48, bt),                                   # blocks differ
        (np.array([40, 30]), 32, bt),                                   # longer than a context
    ]
    for lens, P, table in bad:
        try:
            O.metadata(qsl, lens, P, table, 16)
        except ValueError:
            continue
        raise AssertionError(f"cascade prefix {P} accepted")


def check_cascade_reads_golden(O):
    g = _golden("cascade_reads.json")
    r = O.cascade_prefix_reads(g["R"], g["P"])
    assert r["prefix_naive"] == g["prefix_naive"]
    assert r["prefix_cascade"] == g["prefix_cascade"]
    r2 = O.cascade_prefix_reads(3, 10, [1, 2, 3])
    assert r2["naive"] == 3 * 10 + 6 and r2["cascade"] == 10 + 6


def check_merge_states(O):
    rng = np.random.default_rng(30)
    o = rng.standard_normal((3, 2, 4))
    lam = rng.standard_normal((3, 2))
    om, lm = O.merge_states(o, lam, o, lam)                    # two identical halves
    assert np.max(np.abs(om - o)) < 1e-12 and np.max(np.abs(lm - (lam + math.log(2)))) < 1e-12
    om, lm = O.merge_states(o, lam, rng.standard_normal((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.max(np.abs(om - o)) < 1e-12 and np.max(np.abs(lm - lam)) < 1e-12
    # two single-key parts: weights e^s1 and e^s2
    s1, s2 = 0.7, -1.3
    v1, v2 = rng.standard_normal(4), rng.standard_normal(4)
    om, lm = O.merge_states(v1[None], np.array([s1]), v2[None], np.array([s2]))
    Z = math.exp(s1) + math.exp(s2)
    assert np.max(np.abs(om[0] - (math.exp(s1) * v1 + math.exp(s2) * v2) / Z)) < 1e-12
    assert abs(lm[0] - math.log(Z)) < 1e-12


def check_decode_intensity_golden(O):
    g = _golden("decode_intensity.json")
    r = O.decode_intensity(128, 4096, g["bytes_per_elem"])
    assert abs(r["macs_per_byte_one_product"] - g["macs_per_byte_one_product"]) < 1e-15
    assert abs(r["flop_per_byte"] - 1.0) < 1e-15
    assert abs(O.decode_intensity(128, 4096, 2, group=4)["flop_per_byte"] - 4.0) < 1e-15
    assert abs(O.decode_intensity(128, 4096, 2, group=8)["flop_per_byte"] - 8.0) < 1e-15


def check_bf16_widening(O):
    # bf16 patterns widen exactly: 1.0 = 0x3F80, -2.0 = 0xC000, 0.15625 = 0x3E20,
    # the smallest normal 2^-126 = 0x0080, NaN stays NaN.
    bits = np.array([0x3F80, 0xC000, 0x3E20, 0x0080, 0x7FC0], dtype=np.uint16)
    v = O.to_f64(bits, "bf16")
    assert list(v[:4]) == [1.0, -2.0, 0.15625, 2.0 ** -126] and np.isnan(v[4])


def check_write_kv_fills_pages(O):
    # Whole prompts written token by token through the slot mapping into an
    # all-NaN pool reproduce, bit for bit (NaNs included), the pool that the
    # reshape-based writer builds from the same contiguous K/V and placement.
    for bs, lens in ((16, [1, 15, 16, 17, 50]), (48, [100, 47, 3])):
        Ks, Vs = _random_logical(lens, 2, 8, seed=70 + bs)
        ref, bt = pool_from_logical(Ks, Vs, bs, seed=71 + bs)
        qsl = _qsl(lens)  # every token is new: q_b = L_b, no context
        slots = O.slot_mapping(qsl, lens, bt, bs)
        assert slots.shape == (sum(lens),)
        got = O.write_kv(np.full_like(ref, np.nan), np.concatenate(Ks), np.concatenate(Vs), slots)
        assert np.array_equal(got, ref, equal_nan=True)


def check_write_kv_chunks_follow_context(O):
    # Chunks and decodes: new token i of sequence b is key position c_b + i.
    # Writing fresh rows for the new tokens changes exactly those positions of
    # the gathered sequence; the context rows and every other slot stay put;
    # a token with slot -1 is skipped.
    lens = MIX_L
    Ks, Vs = _random_logical(lens, 2, 8, seed=80)
    pool, bt = pool_from_logical(Ks, Vs, 16, seed=81)
    qsl = _qsl(MIX_Q)
    slots = O.slot_mapping(qsl, lens, bt, 16)
    rng = np.random.default_rng(82)
    T = int(qsl[-1])
    newK = rng.standard_normal((T, 2, 8)).astype(np.float32)
    newV = rng.standard_normal((T, 2, 8)).astype(np.float32)
    skip = 3  # a token of the third sequence is not written
    slots_skip = slots.copy()
    slots_skip[skip] = -1
    out = O.write_kv(pool, newK, newV, slots_skip)
    for b, L in enumerate(lens):
        K, V = O.gather(out, bt[b], L)
        c = L - MIX_Q[b]
        want_K, want_V = Ks[b].copy(), Vs[b].copy()
        for i in range(MIX_Q[b]):
            t = qsl[b] + i
            if t != skip:
                want_K[c + i], want_V[c + i] = newK[t], newV[t]
        assert np.array_equal(K, want_K) and np.array_equal(V, want_V)
    written = np.zeros(pool.shape[:3], dtype=bool)
    for s in slots_skip[slots_skip >= 0]:
        written[s // 16, :, s % 16] = True
    assert np.array_equal(out[~written], pool[~written], equal_nan=True)
    # a lone skipped token leaves the whole pool as it was
    assert np.array_equal(O.write_kv(pool, newK[:1], newV[:1], np.array([-1])), pool, equal_nan=True)


# ---------------------------------------------------------------------------
# FP8 (e4m3) KV cache
# ---------------------------------------------------------------------------

def _code_pool(lens, Hkv, d, seed, bs=16):
    """An e4m3 pool holding random finite codes for each sequence's K/V, placed
    by the reshape-based writer; unused slots hold the NaN code 0x7F.  Returns
    the pool, the block table and the per-sequence code arrays."""
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    Kc = [rng.choice(finite, size=(L, Hkv, d)) for L in lens]
    Vc = [rng.choice(finite, size=(L, Hkv, d)) for L in lens]
    pf, bt = pool_from_logical([k.astype(np.float32) for k in Kc], [v.astype(np.float32) for v in Vc], bs,
                               seed=seed + 1)
    pool = np.where(np.isnan(pf), 0x7F, pf).astype(np.uint8)
    return pool, bt, Kc, Vc


def check_e4m3_decode_library(O):
    # Every code against the float8_e4m3fn dtype of the PyTorch CPU library
    # (the same OCP E4M3 format): equal values, NaN at the same codes (0x7F, 0xFF).
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert list(np.flatnonzero(np.isnan(got))) == [0x7F, 0xFF]
    # closed forms: 1.0, the largest finite 448, the smallest normal and subnormal
    assert O.e4m3_decode([0x38, 0x7E, 0x08, 0x01, 0x80]).tolist() == [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 0.0]


def check_e4m3_encode(O):
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    # every finite value encodes back to its own code (+0 and -0 included)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(finite)), finite)
    # round to nearest, ties to even: PyTorch's float8_e4m3fn conversion on random
    # in-range float32 values and on every midpoint between neighbouring values
    import torch
    rng = np.random.default_rng(90)
    vals = np.sort(O.e4m3_decode(finite[finite < 0x80]))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-0.02, 0.02, 1000), mids, -mids]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)
    # readings: saturation at +-448, NaN -> 0x7F, the sign of zero is kept
    got = O.e4m3_encode(np.array([449.0, 1e9, -1e9, np.nan, -0.0, -2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -10]))
    assert got.tolist() == [0x7E, 0x7E, 0xFE, 0x7F, 0x80, 0x80, 0x00, 0x02]


def check_quantize_divides_in_float32(O):
    # The written code is encode(float32(x / s)): find x, s with x / s just above
    # the tie 1.0625 (between 1.0 = 0x38 and 1.125 = 0x39) but within half a
    # float32 ulp of it, so the float32 quotient is the tie itself and rounds to
    # the even code 0x38, whereas rounding the exact quotient would give 0x39.
    rng = np.random.default_rng(91)
    for _ in range(20000):
        s = np.float32(rng.uniform(1.5, 3.0))
        x = np.float32(np.float32(1.0625) * s)
        for k in range(-3, 4):
            xx = np.nextafter(x, np.float32(np.inf) if k > 0 else np.float32(-np.inf)) if k else x
            exact = float(xx) / float(s)
            if 0 < exact - 1.0625 < 2.0 ** -25 and np.float32(xx) / s == np.float32(1.0625):
                assert O.quantize(xx, s) == 0x38
                assert O.e4m3_encode(exact) == 0x39
                # per-tensor and per-head scales give the same vector
                assert np.array_equal(O.scales_per_head(s, 3), np.full(3, float(s)))
                assert np.array_equal(O.scales_per_head([1, 2, 4], 3), [1.0, 2.0, 4.0])
                return
    raise AssertionError("no test value found")


def check_fp8_attention_reduces_to_fp32(O):
    # With power-of-two scales, code * scale is exact in float32, so attention
    # over the e4m3 pool must equal attention over the float32 pool of those
    # values (the already pinned fp32 definition).  K and V scales differ, and
    # differ per KV head, so a swapped or misapplied scale changes the result.
    lens, qlens = [17, 33, 40, 64], [1, 1, 9, 64]
    Hkv, g, d = 2, 2, 16
    pool, bt, Kc, Vc = _code_pool(lens, Hkv, d, seed=92)
    ks = np.array([2.0 ** -6, 2.0 ** -4], dtype=np.float32)
    vs = np.array([2.0 ** -3, 2.0 ** -7], dtype=np.float32)
    Kf = [(O.e4m3_decode(k) * ks[None, :, None]).astype(np.float32) for k in Kc]
    Vf = [(O.e4m3_decode(v) * vs[None, :, None]).astype(np.float32) for v in Vc]
    pool32, bt2 = pool_from_logical(Kf, Vf, 16, seed=93)
    rng = np.random.default_rng(94)
    q = rng.standard_normal((sum(qlens), Hkv * g, d)).astype(np.float32)
    qb = (q.view(np.uint32) >> np.uint32(16)).astype(np.uint16)       # truncate to bf16 patterns
    q32 = (qb.astype(np.uint32) << np.uint32(16)).view(np.float32)
    out8, lse8 = O.attention(qb, pool, bt, _qsl(qlens), np.array(lens), 0.25, dtype="bf16",
                             kv_dtype="fp8_e4m3", k_scale=ks, v_scale=vs)
    out32, lse32 = O.attention(q32, pool32, bt2, _qsl(qlens), np.array(lens), 0.25, dtype="fp32")
    assert np.abs(out8 - out32).max() < 1e-12 and np.abs(lse8 - lse32).max() < 1e-12
    # the dequantised pool is the same float32 pool up to placement
    deq = O.dequantize_pool(pool, ks, vs)
    for b, L in enumerate(lens):
        K, V = O.gather(deq, bt[b], L)
        assert np.array_equal(K, Kf[b].astype(np.float64)) and np.array_equal(V, Vf[b].astype(np.float64))
    # cascade over the e4m3 pool agrees with the full definition
    P = 32
    cl = [P + 5, P + 20, P + 1]
    poolc, btc, _, _ = _code_pool_shared(cl, Hkv, d, seed=95, prefix_blocks=P // 16)
    qc = (rng.standard_normal((3, Hkv * g, d)).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    full = O.attention(qc, poolc, btc, _qsl([1, 1, 1]), np.array(cl), 0.3, kv_dtype="fp8_e4m3", k_scale=ks, v_scale=vs)
    casc = O.cascade_attention(qc, poolc, btc, _qsl([1, 1, 1]), np.array(cl), 0.3, P, kv_dtype="fp8_e4m3",
                               k_scale=ks, v_scale=vs)
    assert np.abs(full[0] - casc[0]).max() < 1e-12 and np.abs(full[1] - casc[1]).max() < 1e-12


def _code_pool_shared(lens, Hkv, d, seed, prefix_blocks):
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    Kc = [rng.choice(finite, size=(L, Hkv, d)) for L in lens]
    Vc = [rng.choice(finite, size=(L, Hkv, d)) for L in lens]
    pf, bt = pool_from_logical([k.astype(np.float32) for k in Kc], [v.astype(np.float32) for v in Vc], 16,
                               seed=seed + 1, shared_prefix_blocks=prefix_blocks)
    return np.where(np.isnan(pf), 0x7F, pf).astype(np.uint8), bt, Kc, Vc


def check_write_kv_fp8(O):
    # Values that are exactly code * scale (power-of-two per-head scales) written
    # through the slot mapping come back as those codes; values beyond the range
    # saturate; a skipped token and the other slots keep the pool's bytes.
    lens, qlens = [17, 40], [1, 8]
    Hkv, d = 2, 8
    pool, bt, Kc, Vc = _code_pool(lens, Hkv, d, seed=96)
    qsl = _qsl(qlens)
    slots = O.slot_mapping(qsl, lens, bt, 16)
    T = int(qsl[-1])
    rng = np.random.default_rng(97)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    newKc = rng.choice(finite, size=(T, Hkv, d))
    newVc = rng.choice(finite, size=(T, Hkv, d))
    ks = np.array([0.5, 4.0], dtype=np.float32)
    vs = np.array([0.125, 2.0], dtype=np.float32)
    newK = O.e4m3_decode(newKc) * ks[None, :, None]
    newV = O.e4m3_decode(newVc) * vs[None, :, None]
    newK[0, 1, 0] = 1e6                      # saturates to 448 * 4 -> code 0x7E
    slots_skip = slots.copy()
    slots_skip[2] = -1
    out = O.write_kv_fp8(pool, newK, newV, slots_skip, ks, vs)
    want = pool.copy()
    for t, sl in enumerate(slots_skip):
        if sl < 0:
            continue
        want[sl // 16, 0, sl % 16] = newKc[t]
        want[sl // 16, 1, sl % 16] = newVc[t]
    want[slots_skip[0] // 16, 0, slots_skip[0] % 16, 1, 0] = 0x7E
    assert np.array_equal(out, want)
    # one scale for the whole tensor broadcasts to every head
    one = O.write_kv_fp8(pool, newK[:1] * 0 + 3.0, newV[:1] * 0 - 3.0, slots[:1], [2.0], [2.0])
    sl = slots[0]
    assert (one[sl // 16, 0, sl % 16] == 0x3C).all() and (one[sl // 16, 1, sl % 16] == 0xBC).all()


# ---------------------------------------------------------------------------
# Pool memory order (NHD / HND) and large pages
# ---------------------------------------------------------------------------

def _flat_pool(logical, layout):
    """Physical pool for a logical (blocks, 2, bs, Hkv, d) array, written element
    by element at its flat offset: NHD ((blk*2 + kv)*bs + slot)*Hkv*d + h*d + e,
    HND ((blk*2 + kv)*Hkv + h)*bs*d + slot*d + e."""
    nb, _, bs, Hkv, d = logical.shape
    flat = np.empty(logical.size, dtype=logical.dtype)
    for blk in range(nb):
        for kv in range(2):
            for slot in range(bs):
                for h in range(Hkv):
                    if layout == "NHD":
                        off = ((blk * 2 + kv) * bs + slot) * Hkv * d + h * d
                    else:
                        off = ((blk * 2 + kv) * Hkv + h) * bs * d + slot * d
                    flat[off:off + d] = logical[blk, kv, slot, h]
    shape = (nb, 2, bs, Hkv, d) if layout == "NHD" else (nb, 2, Hkv, bs, d)
    return flat.reshape(shape)


def check_layout_gather(O):
    # «FlashAttention y FlashInfer», §Motivación de diseño: NHD keeps the
    # logical order, HND puts the KV head before the slot.
    assert tuple(O.kv_cache_stride_order("NHD")) == (0, 1, 2, 3, 4)
    assert tuple(O.kv_cache_stride_order("HND")) == (0, 1, 3, 2, 4)
    for bs, lens in ((16, [1, 15, 17, 40]), (128, [130, 5, 256])):
        Ks, Vs = _random_logical(lens, 3, 4, seed=100 + bs)
        pool, bt = pool_from_logical(Ks, Vs, bs, seed=101 + bs)
        for layout in ("NHD", "HND"):
            phys = _flat_pool(pool, layout)
            for b, L in enumerate(lens):
                K, V = O.gather(phys, bt[b], L, kv_layout=layout)
                assert np.array_equal(K, Ks[b]) and np.array_equal(V, Vs[b])


def check_layout_attention_and_large_pages(O):
    # The memory order changes nothing in the result; pages of 128 .. 1024
    # tokens (the large pages of «FlashAttention y FlashInfer», §Motivación de
    # diseño) give the same attention as 16-token pages of the same values.
    lens, qlens = [300, 1025, 64, 700], [1, 1, 64, 30]
    Ks, Vs = _random_logical(lens, 2, 8, seed=110)
    rng = np.random.default_rng(111)
    q = rng.standard_normal((sum(qlens), 4, 8)).astype(np.float32)
    ref = None
    for bs in (16, 128, 1024):
        pool, bt = pool_from_logical(Ks, Vs, bs, seed=112 + bs)
        for layout in ("NHD", "HND"):
            phys = _flat_pool(pool, layout)
            got = O.attention(q, phys, bt, _qsl(qlens), np.array(lens), 0.3, dtype="fp32", kv_layout=layout)
            if ref is None:
                ref = got
            assert np.abs(got[0] - ref[0]).max() < 1e-12 and np.abs(got[1] - ref[1]).max() < 1e-12
    # cascade over an HND pool with 128-token pages
    P = 256
    cl = [P + 3, P + 100, P + 129]
    Kc, Vc = _random_logical(cl, 2, 8, seed=113)
    poolc, btc = pool_from_logical(Kc, Vc, 128, seed=114, shared_prefix_blocks=P // 128)
    physc = _flat_pool(poolc, "HND")
    qc = rng.standard_normal((3, 4, 8)).astype(np.float32)
    full = O.attention(qc, physc, btc, _qsl([1, 1, 1]), np.array(cl), 0.3, dtype="fp32", kv_layout="HND")
    casc = O.cascade_attention(qc, physc, btc, _qsl([1, 1, 1]), np.array(cl), 0.3, P, dtype="fp32",
                               kv_layout="HND")
    assert np.abs(full[0] - casc[0]).max() < 1e-12 and np.abs(full[1] - casc[1]).max() < 1e-12


def check_layout_writes(O):
    # Writes into an HND pool land where the flat HND offsets say: the HND
    # result is the flat-offset image of the NHD result (bf16-like float and
    # e4m3 writes alike).
    lens, qlens = [17, 40], [1, 8]
    Ks, Vs = _random_logical(lens, 2, 8, seed=120)
    pool, bt = pool_from_logical(Ks, Vs, 16, seed=121)
    slots = O.slot_mapping(_qsl(qlens), lens, bt, 16)
    rng = np.random.default_rng(122)
    T = sum(qlens)
    nk = rng.standard_normal((T, 2, 8)).astype(np.float32)
    nv = rng.standard_normal((T, 2, 8)).astype(np.float32)
    nhd = O.write_kv(pool, nk, nv, slots)
    hnd = O.write_kv(_flat_pool(pool, "HND"), nk, nv, slots, kv_layout="HND")
    assert np.array_equal(hnd, _flat_pool(nhd, "HND"), equal_nan=True)
    codes = np.where(np.isnan(pool), 0x7F, np.abs(pool * 10) % 120).astype(np.uint8)
    ks, vs = np.array([0.5, 2.0], np.float32), np.array([0.25, 1.0], np.float32)
    nhd8 = O.write_kv_fp8(codes, nk, nv, slots, ks, vs)
    hnd8 = O.write_kv_fp8(_flat_pool(codes, "HND"), nk, nv, slots, ks, vs, kv_layout="HND")
    assert np.array_equal(hnd8, _flat_pool(nhd8, "HND"))
    deq = O.dequantize_pool(_flat_pool(codes, "HND"), ks, vs, kv_layout="HND")
    assert np.array_equal(deq, _flat_pool(O.dequantize_pool(codes, ks, vs), "HND"), equal_nan=True)


ALL_CHECKS = [
    check_kv_cache_shape,
    check_gather_roundtrip,
    check_single_key,
    check_equal_scores,
    check_ramp_needle,
    check_bruteforce_tiny,
    check_sdpa_special_case,
    check_cascade_equals_full,
    check_chunk_consistency,
    check_gqa_expansion,
    check_batch_permutation,
    check_block_permutation,
    check_metadata_golden,
    check_metadata_cascade_errors,
    check_cascade_reads_golden,
    check_merge_states,
    check_decode_intensity_golden,
    check_bf16_widening,
    check_e4m3_decode_library,
    check_e4m3_encode,
    check_quantize_divides_in_float32,
    check_fp8_attention_reduces_to_fp32,
    check_write_kv_fp8,
    check_layout_gather,
    check_layout_attention_and_large_pages,
    check_layout_writes,
    check_write_kv_fills_pages,
    check_write_kv_chunks_follow_context,
]
