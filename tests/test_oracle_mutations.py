"""Plant plausible mistakes in copies of the oracle and check that a pin fails.

Each mutant is the oracle's source with one edit, executed as a fresh module on
the CPU.  The test passes when at least one pin in ``oracle_pins`` rejects the
mutant, showing that the pins constrain that part of the oracle.
"""
import os
import types

import pytest

from tests import oracle_pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE_DIR, "attention.py")
SRC_FP8 = os.path.join(ORACLE_DIR, "fp8.py")
SRC_LAYOUT = os.path.join(ORACLE_DIR, "layout.py")
FP8_IMPORT = "from .fp8 import e4m3_decode, scales_per_head\n"
LAYOUT_IMPORT_ATT = "from .layout import kv_cache_stride_order, logical_pool  # noqa: F401\n"
LAYOUT_IMPORT_FP8 = "from .layout import logical_pool\n"

MUTANTS = {
    "causal_off_by_one": ("visible = t[None, :] <= (cb + i)[:, None]\n        else:\n            visible = np.ones((len(i), Lb)",
                          "visible = t[None, :] < (cb + i)[:, None]\n        else:\n            visible = np.ones((len(i), Lb)"),
    "context_ignores_query_len": ("cb = Lb - qb\n", "cb = Lb - 1\n"),
    "kv_slot_swapped": ("K = kv_cache[blocks, 0, slots]\n    V = kv_cache[blocks, 1, slots]",
                        "K = kv_cache[blocks, 1, slots]\n    V = kv_cache[blocks, 0, slots]"),
    "block_and_slot_swapped": ("[t // bs]\n    slots = t % bs", "[t % bs]\n    slots = t // bs"),
    "gqa_interleaved": ("            heads = slice(kvh * g, (kvh + 1) * g)\n            o, s = _partial(Q[:, heads, :]",
                        "            heads = slice(kvh, H, Hkv)\n            o, s = _partial(Q[:, heads, :]"),
    "lse_base_2": ("lse[has] = m[has] + np.log(l[has])", "lse[has] = m[has] + np.log2(l[has])"),
    "scale_dropped": ("S = scale * (Qg @ K.T)", "S = (Qg @ K.T)"),
    "v_replaced_by_k": ("num = E @ V ", "num = E @ K "),
    "not_normalised": ("o[has] = num[has] / l[has][:, None]", "o[has] = num[has]"),
    "lse_without_max": ("lse[has] = m[has] + np.log(l[has])", "lse[has] = np.log(l[has])"),
    "decode_threshold": ("is_decode = qlen == 1", "is_decode = qlen <= 2"),
    "prefill_first": ("order = np.array(decodes + prefills", "order = np.array(prefills + decodes"),
    "merge_unnormalised": ("o = (w1 / tot_safe)[..., None] * o1 + (w2 / tot_safe)[..., None] * o2",
                           "o = w1[..., None] * o1 + w2[..., None] * o2"),
    "merge_lse_max_only": ("lse = np.where(tot > 0, mx_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)",
                           "lse = np.where(tot > 0, mx_safe, -np.inf)"),
    "cascade_suffix_positions": ("t = np.arange(P, Lb)", "t = np.arange(0, Lb - P)"),
    "cascade_reads_naive": ('"prefix_naive": R * P,', '"prefix_naive": R + P,'),
    "shape_order": ("return (int(num_blocks), 2, int(block_size), int(num_kv_heads), int(head_size))",
                    "return (int(num_blocks), int(block_size), 2, int(num_kv_heads), int(head_size))"),
    "no_block_size_check": ("if block_size % 16 != 0:\n        raise ValueError(\"block size must",
                            "if block_size % 8 != 0:\n        raise ValueError(\"block size must"),
    "bf16_widen_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "intensity_drops_pv": ("flops = g * 4 * L * d", "flops = g * 2 * L * d"),
    "slot_ignores_context": ("pos = (int(L[b]) - qb) + np.arange(qb)", "pos = np.arange(qb)"),
    "slot_position_off_by_one": ("pos = (int(L[b]) - qb) + np.arange(qb)", "pos = (int(L[b]) - qb) + np.arange(1, qb + 1)"),
    "slot_block_offset_swapped": ("bt[b, pos // block_size] * block_size + pos % block_size",
                                  "bt[b, pos % block_size] * block_size + pos // block_size"),
    "write_kv_halves_swapped": ("pool[s // bs, 0, s % bs] = key[t]\n        pool[s // bs, 1, s % bs] = value[t]",
                                "pool[s // bs, 1, s % bs] = key[t]\n        pool[s // bs, 0, s % bs] = value[t]"),
    "write_kv_no_skip": ("        if s < 0:\n            continue\n", ""),
}


# Mutations of the e4m3 module (format, rounding, scales, quantised write) and
# of the attention module's use of it.
MUTANTS_FP8 = {
    "e4m3_bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "e4m3_subnormal_step": ("subnormal = sign * m * 2.0 ** -9", "subnormal = sign * m * 2.0 ** -10"),
    "e4m3_mantissa_bits": ("(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),
    "e4m3_inf_codes_nan": ("(e == 15) & (m == 7)", "(e == 15)"),
    "e4m3_ties_away": ("best = best[codes[best] % 2 == 0]", "best = best[-1:]"),
    "e4m3_nan_saturates": ("            out[n] = 0x7F\n            continue", "            out[n] = 0x7E\n            continue"),
    "e4m3_zero_sign_lost": ("neg = v < 0 or (v == 0 and np.signbit(v))", "neg = v < 0"),
    "quantize_in_float64": ("y = np.asarray(x, dtype=np.float32) / np.float32(scale)\n    return e4m3_encode(y.astype(np.float32))",
                            "y = np.asarray(x, dtype=np.float64) / float(scale)\n    return e4m3_encode(y)"),
    "quantize_multiplies": ("/ np.float32(scale)", "* np.float32(scale)"),
    "per_tensor_scale_ignored": ("return np.full(num_kv_heads, s[0])", "return np.full(num_kv_heads, 1.0)"),
    "dequantize_scales_swapped": ("lv[:, 0] *= ks[None, None, :, None]\n    lv[:, 1] *= vs[None, None, :, None]",
                                  "lv[:, 0] *= vs[None, None, :, None]\n    lv[:, 1] *= ks[None, None, :, None]"),
    "write_fp8_v_with_k_scale": ("quantize(value[t, h], vs[h])", "quantize(value[t, h], ks[h])"),
    "write_fp8_no_skip": ("        if s < 0:\n            continue\n        for h", "        for h"),
    "write_fp8_on_physical_array": ("    pool = logical_pool(out, kv_layout)             # a view: writes land in `out`\n    bs, Hkv",
                                    "    pool = out\n    bs, Hkv"),
}
MUTANTS_ATT_FP8 = {
    "attention_kv_scales_swapped": ("e4m3_decode(K) * ks[None, :, None], e4m3_decode(V) * vs[None, :, None]",
                                    "e4m3_decode(K) * vs[None, :, None], e4m3_decode(V) * ks[None, :, None]"),
    "attention_scale_reversed_heads": ("e4m3_decode(K) * ks[None, :, None]", "e4m3_decode(K) * ks[None, ::-1, None]"),
}
MUTANTS.update(MUTANTS_ATT_FP8)


def _load(src: str, fp8_src: str | None = None, layout_src: str | None = None):
    """The attention module from ``src`` with the e4m3 helpers of ``fp8_src``
    and the memory-order helpers of ``layout_src`` (the real modules' sources
    unless given) in its namespace; the combined namespace also exposes the
    functions of those modules that the pins call."""
    if fp8_src is None:
        with open(SRC_FP8) as f:
            fp8_src = f.read()
    if layout_src is None:
        with open(SRC_LAYOUT) as f:
            layout_src = f.read()
    ml = types.ModuleType("oracle_layout_mutant")
    exec(compile(layout_src, "oracle_layout_mutant", "exec"), ml.__dict__)
    shared = {k: v for k, v in ml.__dict__.items() if not k.startswith("__")}
    m8 = types.ModuleType("oracle_fp8_mutant")
    m8.__dict__.update(shared)
    assert fp8_src.count(LAYOUT_IMPORT_FP8) == 1
    exec(compile(fp8_src.replace(LAYOUT_IMPORT_FP8, ""), "oracle_fp8_mutant", "exec"), m8.__dict__)
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__.update({k: v for k, v in m8.__dict__.items() if not k.startswith("__")})
    assert src.count(FP8_IMPORT) == 1 and src.count(LAYOUT_IMPORT_ATT) == 1
    exec(compile(src.replace(FP8_IMPORT, "").replace(LAYOUT_IMPORT_ATT, ""), "oracle_mutant", "exec"),
         mod.__dict__)
    return mod


def test_unmutated_copy_passes():
    with open(SRC) as f:
        mod = _load(f.read())
    for check in oracle_pins.ALL_CHECKS:
        check(mod)


def _caught(mod):
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:  # any failure (assertion or crash) counts as caught
            failed.append(check.__name__)
    return failed


MUTANTS_LAYOUT = {
    "hnd_is_nhd": ("        return (0, 1, 3, 2, 4)", "        return (0, 1, 2, 3, 4)"),
    "hnd_head_last": ("        return (0, 1, 3, 2, 4)", "        return (0, 1, 2, 4, 3)"),
}
MUTANTS.update({
    "gather_ignores_layout": ("    kv_cache = logical_pool(kv_cache, kv_layout)\n    bs = kv_cache.shape[2]\n    t = np.arange",
                              "    bs = kv_cache.shape[2]\n    t = np.arange"),
    "write_kv_on_physical_array": ("    pool = logical_pool(out, kv_layout)             # a view: writes land in `out`\n    bs = pool.shape[2]\n    for t, s in",
                                   "    pool = out\n    bs = pool.shape[2]\n    for t, s in"),
})


@pytest.mark.parametrize("name", sorted(MUTANTS_LAYOUT))
def test_layout_mutant_is_caught(name):
    old, new = MUTANTS_LAYOUT[name]
    with open(SRC_LAYOUT) as f:
        srcl = f.read()
    assert srcl.count(old) >= 1, f"mutation site for {name} not found"
    with open(SRC) as f:
        mod = _load(f.read(), layout_src=srcl.replace(old, new, 1))
    assert _caught(mod), f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(MUTANTS_FP8))
def test_fp8_mutant_is_caught(name):
    old, new = MUTANTS_FP8[name]
    with open(SRC_FP8) as f:
        src8 = f.read()
    assert src8.count(old) >= 1, f"mutation site for {name} not found"
    with open(SRC) as f:
        mod = _load(f.read(), src8.replace(old, new, 1))
    assert _caught(mod), f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mod = _load(src.replace(old, new, 1))
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:  # any failure (assertion or crash) counts as caught
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
