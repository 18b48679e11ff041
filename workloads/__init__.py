"""Seeded synthetic batches for attention over a paged KV cache.

This module only draws inputs: sequence lengths, a random physical placement of
pages in the pool, and N(0, 1) values for Q, K and V.  It holds none of the
attention arithmetic, so both the CPU oracle and the HIP library can be fed from
it without sharing any computation.

Layout of what it produces (the pool shape is the one the FlashAttention backend
declares in «FlashAttention y FlashInfer», §Flujo de datos):

* ``q``            ``[num_tokens, num_heads, head_size]``
* ``kv_cache``     ``[num_blocks, 2, block_size, num_kv_heads, head_size]``; index 0
                   of dim 1 holds K, index 1 holds V (``kv_layout="HND"`` stores
                   the same pool as ``[num_blocks, 2, num_kv_heads, block_size,
                   head_size]``)
* ``block_table``  int32 ``[num_seqs, max_blocks_per_seq]``
* ``query_start_loc`` int32 ``[num_seqs + 1]``, prefix sums of the query lengths
* ``seq_lens``     int32 ``[num_seqs]``, KV length of each sequence including its
                   new query tokens

bf16 arrays are stored as their raw 16-bit patterns (``np.uint16``) because numpy
has no bfloat16 type; fp32 arrays are ``np.float32``.  An e4m3 pool
(``kv_dtype="fp8_e4m3"``) holds 8-bit codes (``np.uint8``) drawn directly as
random bit fields (sign uniform, exponent field uniform in 5..15, mantissa
uniform, the NaN mantissa 7 of exponent 15 replaced by 6, so codes reach the
largest value 448), with K and V scales drawn per KV head, uniform in
[0.005, 0.007], so the largest value stands for about 3 and the RMS is about
1.3, like the N(0, 1) values of the other pools; no value is quantised here.

Draw order for one batch (each step uses its own child of ``SeedSequence(seed)``):
lengths (drawn by the caller, see ``config_lengths``), page placement, Q, then K/V
page by page.  Pages are filled in fixed chunks, each with its own spawned seed, so
the values do not depend on the number of threads used.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP32_NAN_BITS = np.uint32(0x7FC00000)

_PAGE_CHUNK = 256  # pages per independently seeded chunk of K/V values


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns uint16 bits.

    Input preparation only: the drawn N(0, 1) values are rounded once, and the
    same 16-bit patterns are handed to both sides.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


@dataclass
class Batch:
    """One synthetic batch plus the sizes that describe it."""

    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    dtype: str  # "bf16" | "fp32"
    scale: float
    q: np.ndarray
    kv_cache: np.ndarray
    block_table: np.ndarray
    query_start_loc: np.ndarray
    seq_lens: np.ndarray
    causal: bool = True
    common_prefix_len: int = 0
    name: str = "custom"
    meta: dict = field(default_factory=dict)
    kv_dtype: str = "same"          # "same" or "fp8_e4m3"
    k_scale: np.ndarray | None = None  # e4m3 pool: float32 [num_kv_heads]
    v_scale: np.ndarray | None = None
    kv_layout: str = "NHD"          # memory order of kv_cache: "NHD" or "HND"

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def num_blocks(self) -> int:
        return int(self.kv_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_batch(
    query_lens,
    seq_lens,
    *,
    num_heads: int,
    num_kv_heads: int,
    head_size: int,
    block_size: int,
    dtype: str = "bf16",
    seed: int = 0,
    num_blocks: int | None = None,
    pool_slack: float = 0.10,
    shared_prefix_blocks: int = 0,
    poison: bool = True,
    scale: float | None = None,
    causal: bool = True,
    name: str = "custom",
    max_blocks_per_seq: int | None = None,
    kv_dtype: str = "same",
    kv_layout: str = "NHD",
) -> Batch:
    """Draw a batch for the given per-sequence query lengths and KV lengths.

    ``shared_prefix_blocks`` > 0 places the same physical pages at the front of
    every block-table row (a common prefix).  With ``poison`` the pages that no
    sequence uses, and the slots past each sequence's end in its last page, hold
    NaN, so a kernel that reads them produces NaN.
    """
    if dtype not in ("bf16", "fp32"):
        raise ValueError(f"dtype {dtype!r}")
    if kv_dtype not in ("same", "fp8_e4m3") or (kv_dtype == "fp8_e4m3" and dtype != "bf16"):
        raise ValueError(f"kv_dtype {kv_dtype!r} with dtype {dtype!r}")
    f8 = kv_dtype == "fp8_e4m3"
    qlens = np.asarray(query_lens, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    if qlens.shape != lens.shape:
        raise ValueError("query_lens and seq_lens differ in length")
    B = int(lens.shape[0])
    bs = int(block_size)
    ss = np.random.SeedSequence(seed)
    s_place, s_q, s_kv = ss.spawn(3)

    pages = [(-(-int(L) // bs)) for L in lens]
    sp = int(shared_prefix_blocks)
    if sp and any(p < sp for p in pages):
        raise ValueError("shared prefix longer than a sequence")
    total_pages = sp + sum(p - sp for p in pages)
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil((1.0 + pool_slack) * total_pages)))
    if num_blocks < total_pages:
        raise ValueError("pool too small")
    mbs = max(pages) if pages else 1
    if max_blocks_per_seq is not None:
        if max_blocks_per_seq < mbs:
            raise ValueError("max_blocks_per_seq too small")
        mbs = max_blocks_per_seq

    # (2) physical placement: distinct block ids drawn without replacement
    rng = np.random.Generator(np.random.PCG64(s_place))
    perm = rng.permutation(num_blocks).astype(np.int32)
    pad_id = int(perm[total_pages]) if num_blocks > total_pages else 0
    bt = np.full((B, mbs), pad_id, dtype=np.int32)
    prefix_ids = perm[:sp]
    cursor = sp
    for b, p in enumerate(pages):
        bt[b, :sp] = prefix_ids
        own = p - sp
        bt[b, sp:p] = perm[cursor:cursor + own]
        cursor += own
    used_ids = perm[:total_pages]

    # (3) queries
    T = int(qlens.sum())
    rq = np.random.Generator(np.random.PCG64(s_q))
    qf = rq.standard_normal((T, num_heads, head_size), dtype=np.float32)
    q = f32_to_bf16_bits(qf) if dtype == "bf16" else qf

    # (4) K/V values, page by page in fixed chunks
    shape = (num_blocks, 2, bs, num_kv_heads, head_size)
    if f8:
        pool = np.empty(shape, dtype=np.uint8)
        fill = np.uint8(0x7F) if poison else np.uint8(0)
    elif dtype == "bf16":
        pool = np.empty(shape, dtype=np.uint16)
        fill = BF16_NAN if poison else np.uint16(0)
    else:
        pool = np.empty(shape, dtype=np.float32)
        fill = np.float32(np.nan) if poison else np.float32(0)
    n_chunks = -(-total_pages // _PAGE_CHUNK)
    kids = s_kv.spawn(max(n_chunks, 1))

    def fill_chunk(ci: int) -> None:
        ids = used_ids[ci * _PAGE_CHUNK:(ci + 1) * _PAGE_CHUNK]
        g = np.random.Generator(np.random.PCG64(kids[ci]))
        if f8:
            fshape = (len(ids),) + shape[1:]
            sign = g.integers(0, 2, size=fshape, dtype=np.uint8)
            expo = g.integers(5, 16, size=fshape, dtype=np.uint8)
            mant = g.integers(0, 8, size=fshape, dtype=np.uint8)
            mant = np.where((expo == 15) & (mant == 7), np.uint8(6), mant)
            pool[ids] = (sign << np.uint8(7)) | (expo << np.uint8(3)) | mant
            return
        vals = g.standard_normal((len(ids),) + shape[1:], dtype=np.float32)
        pool[ids] = f32_to_bf16_bits(vals) if dtype == "bf16" else vals

    unused = np.sort(perm[total_pages:])
    pool[unused] = fill
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill_chunk, range(n_chunks)))

    # stale slots past the end of each sequence's last page
    if poison:
        for b, L in enumerate(lens):
            tail = int(L) % bs
            if tail and pages[b] > sp:
                pool[bt[b, pages[b] - 1], :, tail:] = fill

    qsl = np.zeros(B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(qlens)
    if kv_layout == "HND":   # store the same logical pool with the KV head before the slot
        pool = np.ascontiguousarray(pool.transpose(0, 1, 3, 2, 4))
    elif kv_layout != "NHD":
        raise ValueError(f"kv_layout {kv_layout!r}")
    k_scale = v_scale = None
    if f8:
        rs = np.random.Generator(np.random.PCG64(ss.spawn(1)[0]))
        k_scale = rs.uniform(0.005, 0.007, size=num_kv_heads).astype(np.float32)
        v_scale = rs.uniform(0.005, 0.007, size=num_kv_heads).astype(np.float32)
    return Batch(
        num_heads=num_heads,
        num_kv_heads=num_kv_heads,
        head_size=head_size,
        block_size=bs,
        dtype=dtype,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(head_size)),
        q=q,
        kv_cache=pool,
        block_table=bt,
        query_start_loc=qsl,
        seq_lens=lens.astype(np.int32),
        causal=causal,
        common_prefix_len=sp * bs,
        name=name,
        meta={"pad_block_id": pad_id, "total_pages": total_pages, "seed": seed},
        kv_dtype=kv_dtype,
        k_scale=k_scale,
        v_scale=v_scale,
        kv_layout=kv_layout,
    )


# ---------------------------------------------------------------------------
# The five workload shapes.  Configuration 1 is fixed; 2-5 draw their lengths
# from a PCG64 stream seeded with the configuration number.  Shape 6 is an
# extra beyond the five: the cascade batch with four 512-token prefill chunks
# that share its prefix (a shared-prefix step with decodes and prefills).
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny_mixed",
    2: "decode_only",
    3: "prefill_causal_varlen",
    4: "chunked_prefill_mixed",
    5: "cascade_shared_prefix",
    6: "cascade_shared_prefix_with_chunks",
}

CONFIG_SHAPES = {
    1: dict(num_heads=4, num_kv_heads=2, head_size=64, block_size=16, dtype="fp32"),
    2: dict(num_heads=32, num_kv_heads=8, head_size=128, block_size=16, dtype="bf16"),
    3: dict(num_heads=32, num_kv_heads=8, head_size=128, block_size=16, dtype="bf16"),
    4: dict(num_heads=64, num_kv_heads=8, head_size=128, block_size=64, dtype="bf16"),
    5: dict(num_heads=32, num_kv_heads=8, head_size=128, block_size=16, dtype="bf16"),
    6: dict(num_heads=32, num_kv_heads=8, head_size=128, block_size=16, dtype="bf16"),
}


def config_lengths(cfg: int, seed: int | None = None):
    """Query lengths, KV lengths and shared-prefix page count of a configuration."""
    seed = cfg if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(1)[0]))
    if cfg == 1:
        # 2 decodes, 1 chunk with 48 context tokens, 1 full causal prefill
        return np.array([1, 1, 16, 100]), np.array([17, 33, 64, 100]), 0
    if cfg == 2:
        L = rng.integers(512, 8192, size=256, endpoint=True)
        return np.ones(256, dtype=np.int64), L, 0
    if cfg == 3:
        L = rng.integers(512, 4096, size=16, endpoint=True)
        return L.copy(), L, 0
    if cfg == 4:
        Ld = rng.integers(1024, 16384, size=192, endpoint=True)
        ctx = rng.integers(2048, 8192, size=4, endpoint=True)
        q = np.concatenate([np.ones(192, dtype=np.int64), np.full(4, 512)])
        return q, np.concatenate([Ld, ctx + 512]), 0
    if cfg == 5:
        P = 16384
        s = rng.integers(256, 2048, size=128, endpoint=True)
        return np.ones(128, dtype=np.int64), P + s, P // 16
    if cfg == 6:
        # the cascade batch's decodes, then 4 chunks of 512 queries whose
        # context is the shared prefix plus 256..2048 tokens of their own
        P = 16384
        s = rng.integers(256, 2048, size=128, endpoint=True)
        own = rng.integers(256, 2048, size=4, endpoint=True)
        q = np.concatenate([np.ones(128, dtype=np.int64), np.full(4, 512)])
        return q, np.concatenate([P + s, P + own + 512]), P // 16
    raise ValueError(f"unknown configuration {cfg}")


def config_batch(cfg: int, seed: int | None = None, poison: bool = True, kv_dtype: str = "same",
                 kv_layout: str = "NHD", block_size: int | None = None) -> Batch:
    """Draw the full-size batch of configuration ``cfg`` (1..5, or the extra
    shape 6); ``kv_dtype``
    "fp8_e4m3" gives the same lengths and placement over an e4m3 pool."""
    seed = cfg if seed is None else seed
    qlens, lens, sp = config_lengths(cfg, seed)
    shape = dict(CONFIG_SHAPES[cfg])
    if block_size is not None:  # same lengths and values, other page size
        shape["block_size"] = int(block_size)
    kw = {}
    if cfg == 1:
        kw["num_blocks"] = 64
        kw["scale"] = 1.0 / 8.0
    return make_batch(
        qlens, lens, seed=seed, shared_prefix_blocks=sp, poison=poison,
        name=CONFIG_NAMES[cfg], kv_dtype=kv_dtype, kv_layout=kv_layout, **shape, **kw,
    )
