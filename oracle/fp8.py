"""8-bit e4m3 floating point for the KV cache (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline may
import this module.

The pages name an FP8 KV cache (``fp8`` / ``fp8_e4m3``) and per-head
quantisation scales («FlashAttention y FlashInfer», §Motivación de diseño and
§Límites y fallos; «El especialista del plato estrella», §Los 10 knobs, the
``kv_cache_dtype`` row, and §Cómo se conecta con el resto del stack;
«AttentionBackend: capa de abstracción», §Límites y fallos) but print no
formula.  Readings taken here:

* The format is the OCP 8-bit "E4M3" float: 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
  ``m * 2**-9``; there are no infinities, and only the two codes with every
  exponent and mantissa bit set (0x7F, 0xFF) are NaN, so the largest finite
  magnitude is ``1.75 * 2**8 = 448``.
* A cache entry stands for ``decode(code) * scale``, with one scale for the
  whole K (or V) tensor or one per KV head.
* Writing a value ``x`` stores ``encode(x / scale)``: the division is done in
  float32 (the element type the library computes in), then rounded to the
  nearest e4m3 value, ties to the even code, saturating at +-448; NaN stays NaN.
"""
from __future__ import annotations

import numpy as np

from .layout import logical_pool

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of every e4m3 code (NaN for 0x7F and 0xFF), by the format's
    definition: sign, biased exponent and mantissa fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e - 7.0)
    subnormal = sign * m * 2.0 ** -9
    v = np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def _positive_table():
    """The 127 non-negative finite e4m3 values, ascending, with their codes 0x00..0x7E."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return e4m3_decode(codes), codes


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each value (ties to the even code, i.e. the one whose
    lowest mantissa bit is 0), saturating at +-448; NaN -> 0x7F; the sign of a
    zero result is the sign of the input.  Found by comparing against every
    finite value of the format (no bit tricks)."""
    xa = np.asarray(x, dtype=np.float64)
    flat = xa.reshape(-1)
    vals, codes = _positive_table()
    out = np.empty(flat.shape, dtype=np.uint8)
    for n, v in enumerate(flat):
        if np.isnan(v):
            out[n] = 0x7F
            continue
        a = min(abs(v), E4M3_MAX)
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:                       # an exact tie between two neighbours
            best = best[codes[best] % 2 == 0]
        code = int(codes[best[0]])
        neg = v < 0 or (v == 0 and np.signbit(v))
        out[n] = code | (0x80 if neg else 0)
    return out.reshape(xa.shape)


def quantize(x, scale) -> np.ndarray:
    """Codes written for values ``x`` (float32-exact, e.g. bf16) with a positive
    ``scale``: ``encode(float32(x) / float32(scale))``, the division in float32."""
    y = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return e4m3_encode(y.astype(np.float32))


def scales_per_head(scale, num_kv_heads: int) -> np.ndarray:
    """A per-tensor scale (one value) or per-head scales (``num_kv_heads``
    values) as a float64 vector of one entry per KV head."""
    s = np.asarray(scale, dtype=np.float32).reshape(-1).astype(np.float64)
    if s.size == 1:
        return np.full(num_kv_heads, s[0])
    if s.size != num_kv_heads:
        raise ValueError("one scale, or one per KV head")
    return s


def dequantize_pool(kv_cache, k_scale, v_scale, kv_layout: str = "NHD") -> np.ndarray:
    """float64 pool of an e4m3 pool, same shape and memory order: K entries are
    ``decode(code) * k_scale[kvh]`` and V entries ``decode(code) * v_scale[kvh]``."""
    pool = np.asarray(kv_cache, dtype=np.uint8)
    out = e4m3_decode(pool)
    lv = logical_pool(out, kv_layout)               # a view of `out`
    Hkv = lv.shape[3]
    ks = scales_per_head(k_scale, Hkv)
    vs = scales_per_head(v_scale, Hkv)
    lv[:, 0] *= ks[None, None, :, None]
    lv[:, 1] *= vs[None, None, :, None]
    return out


def write_kv_fp8(kv_cache, key, value, slots, k_scale, v_scale, kv_layout: str = "NHD"):
    """A copy of an e4m3 pool with token ``t``'s K and V rows quantised with the
    K / V scale of each KV head and stored at slot ``slots[t]`` (block ``s // bs``,
    offset ``s % bs``); a negative slot skips the token.  ``key`` and ``value``
    are ``[T, Hkv, d]`` arrays of values (not bit patterns) that float32 holds
    exactly, e.g. the values of bf16 inputs."""
    out = np.array(kv_cache, dtype=np.uint8, copy=True)
    pool = logical_pool(out, kv_layout)             # a view: writes land in `out`
    bs, Hkv = pool.shape[2], pool.shape[3]
    ks = scales_per_head(k_scale, Hkv)
    vs = scales_per_head(v_scale, Hkv)
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        for h in range(Hkv):
            pool[s // bs, 0, s % bs, h] = quantize(key[t, h], ks[h])
            pool[s // bs, 1, s % bs, h] = quantize(value[t, h], vs[h])
    return out
