"""Plain float64 definition of paged-KV varlen attention (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline may
import this module.  See the package docstring for the pages it follows.

Notation (per sequence ``b`` of a batch of ``B``): ``q_b`` query tokens, KV length
``L_b = seq_lens[b]`` (it includes the new query tokens), context ``c_b = L_b - q_b``,
``H`` query heads, ``Hkv`` KV heads, group ``g = H / Hkv``, head size ``d``,
block size ``bs``.  Query ``i`` of sequence ``b`` sits at position ``c_b + i``.

Readings taken where the pages leave a step open:

* ``seq_lens`` counts the new query tokens, so ``c_b = L_b - q_b``.
* Causal masking is aligned to the end of the KV: query ``i`` sees keys
  ``0 .. c_b + i``.  A decode (``q_b = 1``) therefore sees all ``L_b`` keys, which
  is the "one query against all the accumulated KV" of the decode description.
* Query head ``h`` reads KV head ``h // g`` (consecutive query heads share one KV
  head).
* A sequence is a decode when it brings exactly one query token.
* The log-sum-exp is the natural logarithm of the sum of exponentiated scaled
  scores.
"""
from __future__ import annotations

import numpy as np

from .fp8 import e4m3_decode, scales_per_head
from .layout import kv_cache_stride_order, logical_pool  # noqa: F401


# ---------------------------------------------------------------------------
# Pool shape and element conversion
# ---------------------------------------------------------------------------

def kv_cache_shape(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int):
    """Shape of the paged pool.

    «FlashAttention y FlashInfer», §Flujo de datos (``get_kv_cache_shape`` listing):
    the pool is (blocks, K/V slot, slots per block, KV heads, head size), and a
    block size that is not a multiple of 16 is rejected.
    """
    if block_size % 16 != 0:
        raise ValueError("block size must be a multiple of 16")
    return (int(num_blocks), 2, int(block_size), int(num_kv_heads), int(head_size))


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening to float64.

    bf16 values arrive as their 16-bit patterns; a bfloat16 is the upper half of
    the float32 with the same value, so shifting the pattern left by 16 bits gives
    that float32 exactly, and float32 -> float64 is exact too.
    """
    if dtype == "bf16":
        wide = np.asarray(x).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Batch metadata
# ---------------------------------------------------------------------------

def metadata(query_start_loc, seq_lens, common_prefix_len: int = 0,
             block_table=None, block_size: int | None = None) -> dict:
    """Split decodes from prefills and order the batch decode-first.

    «FlashAttention y FlashInfer», §Responsabilidades and the closing paragraph
    of §Flujo de datos: the FlashInfer builder separates decodes from prefills
    and moves the decodes to the front, so that the decode kernel sees one
    contiguous run of equal-length queries.  The order kept inside each group is
    the batch order (a stable partition).

    Cascade («El especialista del plato estrella», §Qué aporta FlashInfer): the
    prefix of ``common_prefix_len`` tokens must be whole blocks, pure context of
    every sequence, and the same physical blocks in every block-table row.
    """
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    qlen = qsl[1:] - qsl[:-1]
    ctx = L - qlen
    is_decode = qlen == 1
    decodes = [b for b in range(len(L)) if is_decode[b]]
    prefills = [b for b in range(len(L)) if not is_decode[b]]
    order = np.array(decodes + prefills, dtype=np.int64)
    md = {
        "query_lens": qlen,
        "context_lens": ctx,
        "is_decode": is_decode,
        "is_chunked": (~is_decode) & (ctx > 0),
        "order": order,
        "num_decodes": len(decodes),
        "num_decode_tokens": int(sum(qlen[b] for b in decodes)),
        "num_prefills": len(prefills),
        "num_prefill_tokens": int(sum(qlen[b] for b in prefills)),
        "num_tokens": int(qsl[-1]) if len(qsl) else 0,
        "common_prefix_len": int(common_prefix_len),
        "prefix_blocks": np.zeros(0, dtype=np.int64),
    }
    P = int(common_prefix_len)
    if P:
        if block_table is None or block_size is None:
            raise ValueError("cascade needs the block table and block size")
        if P % block_size != 0:
            raise ValueError("common prefix must be whole blocks")
        if np.any(ctx < P):
            raise ValueError("common prefix must be context of every sequence")
        bt = np.asarray(block_table)
        nb = P // block_size
        first = bt[0, :nb]
        if np.any(bt[:, :nb] != first[None, :]):
            raise ValueError("common prefix blocks differ between sequences")
        md["prefix_blocks"] = first.astype(np.int64)
    return md


# ---------------------------------------------------------------------------
# Gather
# ---------------------------------------------------------------------------

def gather(kv_cache: np.ndarray, block_table_row, seq_len: int, kv_layout: str = "NHD"):
    """Contiguous K and V of one sequence, ``[seq_len, Hkv, d]`` each, same dtype.

    «El especialista del plato estrella», §Cómo lee el backend el KV paginado:
    the kernel is handed the block table and gathers over the physical blocks.
    Token ``t`` lives in block ``block_table_row[t // bs]`` at slot ``t % bs``;
    slot 0 of the pool's second dimension holds K and slot 1 holds V
    («FlashAttention y FlashInfer», §Flujo de datos).  ``kv_layout`` is the
    pool's memory order (:func:`oracle.layout.kv_cache_stride_order`).
    """
    kv_cache = logical_pool(kv_cache, kv_layout)
    bs = kv_cache.shape[2]
    t = np.arange(int(seq_len))
    blocks = np.asarray(block_table_row, dtype=np.int64)[t // bs]
    slots = t % bs
    K = kv_cache[blocks, 0, slots]
    V = kv_cache[blocks, 1, slots]
    return K, V


# ---------------------------------------------------------------------------
# Cache write
# ---------------------------------------------------------------------------

def slot_mapping(query_start_loc, seq_lens, block_table, block_size: int):
    """Pool slot of every new token, in token order (``int64[T]``).

    «FlashAttention y FlashInfer», §Responsabilidades: putting the new tokens'
    K/V into the paged cache is an operation of its own, separate from the
    attention forward.  Query token ``i`` of sequence ``b`` is key position
    ``c_b + i``; it is stored where the gather reads that position: block
    ``block_table[b][(c_b + i) // bs]`` at offset ``(c_b + i) % bs``.  The slot
    number is ``block * bs + offset``.
    """
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    out = np.empty(int(qsl[-1]) if len(qsl) else 0, dtype=np.int64)
    for b in range(len(L)):
        qb = int(qsl[b + 1] - qsl[b])
        pos = (int(L[b]) - qb) + np.arange(qb)
        out[qsl[b]:qsl[b + 1]] = bt[b, pos // block_size] * block_size + pos % block_size
    return out


def write_kv(kv_cache: np.ndarray, key: np.ndarray, value: np.ndarray, slots, kv_layout: str = "NHD"):
    """A copy of the pool with token ``t``'s K row ``key[t]`` (``[Hkv, d]``) at slot
    ``slots[t]`` of the K half and its V row in the V half; a negative slot skips
    the token.  Slot ``s`` is block ``s // bs``, offset ``s % bs``.  The copy keeps
    the pool's memory order ``kv_layout``.
    """
    out = np.array(kv_cache, copy=True)
    pool = logical_pool(out, kv_layout)             # a view: writes land in `out`
    bs = pool.shape[2]
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        pool[s // bs, 0, s % bs] = key[t]
        pool[s // bs, 1, s % bs] = value[t]
    return out


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _partial(Qg: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, visible: np.ndarray):
    """Softmax attention of ``Qg [n, g, d]`` over keys ``K, V [L, d]``.

    ``visible [n, L]`` says which keys each query row may see.  Returns the
    normalised output ``[n, g, d]`` and the natural-log log-sum-exp ``[n, g]``.
    A row with no visible key has output 0 and log-sum-exp -inf.
    """
    n, g, d = Qg.shape
    S = scale * (Qg @ K.T)                                   # [n, g, L]
    S = np.where(visible[:, None, :], S, -np.inf)
    m = S.max(axis=-1) if S.shape[-1] else np.full((n, g), -np.inf)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    E = np.exp(S - m_safe[..., None])                        # masked entries -> 0
    l = E.sum(axis=-1)
    o = np.zeros((n, g, d))
    num = E @ V                                              # [n, g, d]
    o[has] = num[has] / l[has][:, None]
    lse = np.full((n, g), -np.inf)
    lse[has] = m[has] + np.log(l[has])
    return o, lse


def _dims(q: np.ndarray, kv_cache: np.ndarray):
    H = q.shape[1]
    Hkv = kv_cache.shape[3]
    if H % Hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    return H, Hkv, H // Hkv


def _kv_values(K, V, dtype: str, kv_dtype, k_scale, v_scale):
    """Exact float64 values of gathered K/V rows ``[L, Hkv, d]``: the pool's
    element type, or e4m3 codes times their K / V scale (one per KV head or one
    for the tensor; see :mod:`oracle.fp8`)."""
    if kv_dtype in (None, "same"):
        return to_f64(K, dtype), to_f64(V, dtype)
    if kv_dtype != "fp8_e4m3":
        raise ValueError(f"kv_dtype {kv_dtype!r}")
    Hkv = K.shape[1]
    ks = scales_per_head(k_scale, Hkv)
    vs = scales_per_head(v_scale, Hkv)
    return e4m3_decode(K) * ks[None, :, None], e4m3_decode(V) * vs[None, :, None]


def attention_rows(q, kv_cache, block_table, query_start_loc, seq_lens, scale, rows,
                   *, dtype: str = "bf16", causal: bool = True, kv_dtype=None, k_scale=1.0, v_scale=1.0,
                   kv_layout: str = "NHD"):
    """Output and log-sum-exp of the chosen token rows only (any order).

    Same definition as :func:`attention`; used where the whole batch is too large
    for the CPU.  Returns ``out [len(rows), H, d]`` and ``lse [len(rows), H]``.
    """
    kv_cache = logical_pool(kv_cache, kv_layout)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    H, Hkv, g = _dims(q, kv_cache)
    d = q.shape[2]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), H, d))
    lse = np.zeros((len(rows), H))
    seq_of = np.searchsorted(qsl, rows, side="right") - 1
    for b in np.unique(seq_of):
        sel = np.nonzero(seq_of == b)[0]
        Lb = int(L[b])
        qb = int(qsl[b + 1] - qsl[b])
        cb = Lb - qb
        i = rows[sel] - qsl[b]                                # query index in the sequence
        K, V = gather(kv_cache, block_table[b], Lb)
        K, V = _kv_values(K, V, dtype, kv_dtype, k_scale, v_scale)
        t = np.arange(Lb)
        if causal:
            visible = t[None, :] <= (cb + i)[:, None]
        else:
            visible = np.ones((len(i), Lb), dtype=bool)
        Q = to_f64(q[rows[sel]], dtype)                       # [n, H, d]
        for kvh in range(Hkv):
            heads = slice(kvh * g, (kvh + 1) * g)
            o, s = _partial(Q[:, heads, :], K[:, kvh, :], V[:, kvh, :], scale, visible)
            out[sel, heads, :] = o
            lse[sel, heads] = s
    return out, lse


def attention(q, kv_cache, block_table, query_start_loc, seq_lens, scale,
              *, dtype: str = "bf16", causal: bool = True, kv_dtype=None, k_scale=1.0, v_scale=1.0,
              kv_layout: str = "NHD"):
    """Exact attention for every token row of a mixed varlen batch.

    For row ``r = query_start_loc[b] + i``, head ``h`` and KV head ``h // g``, the
    scores against the gathered keys are ``scale * q . k_t``; the visible set is
    ``t <= c_b + i`` (causal) or all ``t < L_b``; the output is the softmax-
    weighted mean of the visible V rows and the log-sum-exp is
    ``log(sum_t exp(score_t))``.  Prefill rows («El especialista del plato
    estrella», §Por qué prefill y decode son problemas opuestos: many queries
    against many keys) and decode rows (one query against the whole KV) follow
    the same definition; only the number of rows differs.

    With ``kv_dtype="fp8_e4m3"`` the pool holds e4m3 codes and the keys and
    values are ``decode(code) * k_scale`` and ``decode(code) * v_scale`` (one scale,
    or one per KV head); queries keep ``dtype``.  ``kv_layout`` is the pool's
    memory order (NHD or HND).

    Returns ``out [T, H, d]`` and ``lse [T, H]`` in float64, rows in the
    caller's order.
    """
    T = int(np.asarray(query_start_loc)[-1])
    return attention_rows(q, kv_cache, block_table, query_start_loc, seq_lens, scale,
                          np.arange(T), dtype=dtype, causal=causal, kv_dtype=kv_dtype,
                          k_scale=k_scale, v_scale=v_scale, kv_layout=kv_layout)


def merge_states(o1, lse1, o2, lse2):
    """Combine two partial attentions over disjoint key sets by their log-sum-exp.

    «AttentionBackend: capa de abstracción», §Motivación de diseño and §Límites y
    fallos: partial softmax results are combined through the LSE, and the LSE
    base must be consistent.  With natural logs: ``lse = log(e^lse1 + e^lse2)``
    and ``o = e^(lse1 - lse) o1 + e^(lse2 - lse) o2``.  A part over an empty key
    set (lse = -inf) contributes nothing.
    """
    o1 = np.asarray(o1, dtype=np.float64)
    o2 = np.asarray(o2, dtype=np.float64)
    lse1 = np.asarray(lse1, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    mx = np.maximum(lse1, lse2)
    mx_safe = np.where(np.isfinite(mx), mx, 0.0)
    w1 = np.exp(lse1 - mx_safe)
    w2 = np.exp(lse2 - mx_safe)
    tot = w1 + w2
    lse = np.where(tot > 0, mx_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    tot_safe = np.where(tot > 0, tot, 1.0)
    o = (w1 / tot_safe)[..., None] * o1 + (w2 / tot_safe)[..., None] * o2
    return o, lse


def cascade_attention(q, kv_cache, block_table, query_start_loc, seq_lens, scale,
                      common_prefix_len: int, *, dtype: str = "bf16", causal: bool = True,
                      kv_dtype=None, k_scale=1.0, v_scale=1.0, kv_layout: str = "NHD"):
    """Cascade form: shared prefix once, each sequence's own suffix, merged by LSE.

    «El especialista del plato estrella», §Qué aporta FlashInfer: when the batch
    shares a prefix of ``P`` tokens, attention over the prefix is computed once
    for all query rows and combined with each request's attention over its own
    suffix.  All query rows lie after the prefix, so the prefix part is not
    masked; the suffix part keeps the causal mask on keys ``P .. L_b - 1``.
    Returns the same ``out, lse`` as :func:`attention`.
    """
    P = int(common_prefix_len)
    kv_cache = logical_pool(kv_cache, kv_layout)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    bs = kv_cache.shape[2]
    md = metadata(qsl, L, P, block_table, bs)
    H, Hkv, g = _dims(q, kv_cache)
    d = q.shape[2]
    T = int(qsl[-1])
    Qall = to_f64(q, dtype)

    # prefix: every query row of the batch against keys 0 .. P-1
    Kp, Vp = gather(kv_cache, md["prefix_blocks"], P)
    Kp, Vp = _kv_values(Kp, Vp, dtype, kv_dtype, k_scale, v_scale)
    o1 = np.zeros((T, H, d))
    l1 = np.full((T, H), -np.inf)
    vis_p = np.ones((T, P), dtype=bool)
    for kvh in range(Hkv):
        heads = slice(kvh * g, (kvh + 1) * g)
        o, s = _partial(Qall[:, heads, :], Kp[:, kvh, :], Vp[:, kvh, :], scale, vis_p)
        o1[:, heads, :] = o
        l1[:, heads] = s

    # suffix: each sequence's keys P .. L_b - 1
    o2 = np.zeros((T, H, d))
    l2 = np.full((T, H), -np.inf)
    for b in range(len(L)):
        Lb = int(L[b])
        r0, r1 = int(qsl[b]), int(qsl[b + 1])
        cb = Lb - (r1 - r0)
        K, V = gather(kv_cache, block_table[b], Lb)
        K, V = _kv_values(K[P:], V[P:], dtype, kv_dtype, k_scale, v_scale)
        t = np.arange(P, Lb)
        i = np.arange(r1 - r0)
        if causal:
            visible = t[None, :] <= (cb + i)[:, None]
        else:
            visible = np.ones((r1 - r0, Lb - P), dtype=bool)
        for kvh in range(Hkv):
            heads = slice(kvh * g, (kvh + 1) * g)
            o, s = _partial(Qall[r0:r1, heads, :], K[:, kvh, :], V[:, kvh, :], scale, visible)
            o2[r0:r1, heads, :] = o
            l2[r0:r1, heads] = s
    return merge_states(o1, l1, o2, l2)


def cascade_prefix_reads(num_requests: int, prefix_len: int, suffix_lens=None) -> dict:
    """Token reads of the naive and the cascade schedule.

    «El especialista del plato estrella», §Qué aporta FlashInfer (eq. "lecturas"):
    the naive schedule reads the shared prefix once per request, cascade reads it
    once.  Reading of the damaged formula: naive = sum_i (P + s_i) = R*P + sum s_i,
    cascade = P + sum s_i.  ``prefix_*`` are the prefix parts alone.
    """
    s = 0 if suffix_lens is None else int(np.sum(suffix_lens))
    R, P = int(num_requests), int(prefix_len)
    return {
        "prefix_naive": R * P,
        "prefix_cascade": P,
        "naive": R * P + s,
        "cascade": P + s,
    }


def decode_intensity(head_size: int, seq_len: int, bytes_per_elem: int, group: int = 1) -> dict:
    """Arithmetic intensity of one decode step against ``seq_len`` cached keys.

    «El especialista del plato estrella», §Por qué prefill y decode son problemas
    opuestos (eq. I_decode): work grows like ``L d``, bytes like ``L d s``.  Exact
    count for ``group`` query heads sharing one KV head: QK^T and P.V are
    ``2 L d`` flops each per query head; K and V are ``2 L d s`` bytes read once.
    ``macs_per_byte_one_product`` is the page's own convention (one product's
    multiply-adds per byte of one of K or V): ``1/s``.
    """
    L, d, s, g = int(seq_len), int(head_size), int(bytes_per_elem), int(group)
    flops = g * 4 * L * d
    nbytes = 2 * L * d * s
    return {
        "flops": flops,
        "bytes": nbytes,
        "flop_per_byte": flops / nbytes,
        "macs_per_byte_one_product": (L * d) / (L * d * s),
    }
