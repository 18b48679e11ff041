#!/usr/bin/env python3
"""Throughput of libpagedattn on one MI355X, against the chip's roofline.

A step is one pa_forward over one batch (every kernel the batch needs: cascade
prefix pass, decode, prefill, LSE merge), inputs already resident in HBM.

Default workload: decode-only, 256 sequences with context lengths drawn
uniformly from [512, 8192], 32 query / 8 KV heads, head size 128, block size 16,
bf16 (the decode half of the metric); the line also carries a secondary
measurement of the causal varlen prefill workload (16 prompts of 512..4096
tokens, same heads) for the prefill half of the metric.  Other workloads:
``--workload prefill | mixed | cascade | tiny | decode_e4m3 | kvwrite``
(decode_e4m3: the decode batch over a pool of 8-bit e4m3 codes with per-head
K/V scales; its algorithmic bytes count one byte per element).

Prints ONE JSON line.  Algorithmic work counts each KV byte once per KV head
(decode) and 4*H*d FLOPs per visible (query, key) pair (prefill); masked and
skipped work is not counted.  ``roofline.achieved`` divides that by the
dominant kernel's average launch duration, measured with HIP events recorded
on the launch stream by the library (pa_profile_start/stop) over a pass of the
same number of steps run right after the timed one: those records sit between
the launches of a step and would lengthen it, so the timed steps go without.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}  # dense MFMA
METRIC = "decode KV-read GB/s (% HBM peak) + prefill attn TFLOPS (% MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SRC = os.path.join(ROOT, "attention_paged_kv_varlen_amd", "csrc", "kernels.hip")

WORKLOADS = {
    "decode": 2,
    "prefill": 3,
    "mixed": 4,
    "cascade": 5,
    "tiny": 1,
    "decode_e4m3": 2,
    "cascade_chunks": 6,
}
KV_DTYPES = {"decode_e4m3": "fp8_e4m3"}
DESCRIPTIONS = {
    1: "tiny mixed: 4 seqs, seq_lens 17/33/64/100, query_lens 1/1/16/100; 4 q / 2 kv heads, d=64, bs=16, fp32",
    2: "decode-only: 256 seqs, q=1, ctx U[512,8192]; 32 q / 8 kv heads, d=128, bs=16, bf16, random page placement",
    3: "prefill causal varlen: 16 prompts U[512,4096], no context; 32 q / 8 kv heads, d=128, bs=16, bf16",
    4: "chunked-prefill mixed: 192 decodes ctx U[1024,16384] + 4 chunks of 512 with ctx U[2048,8192]; "
       "64 q / 8 kv heads, d=128, bs=64, bf16, decode-first",
    5: "cascade: 128 decodes sharing a 16384-token prefix + suffixes U[256,2048]; 32 q / 8 kv heads, d=128, "
       "bs=16, bf16",
    6: "cascade with chunks: the cascade batch plus 4 chunks of 512 sharing its prefix (own context "
       "U[256,2048]); 32 q / 8 kv heads, d=128, bs=16, bf16",
}


# ---------------------------------------------------------------------------
# Algorithmic counts
# ---------------------------------------------------------------------------

def algorithmic_counts(query_lens, seq_lens, *, num_heads, num_kv_heads, head_size, elem_bytes,
                       common_prefix_len=0, causal=True) -> dict:
    """Bytes and FLOPs the method needs, independent of how a kernel does it.

    decode_bytes: K and V of every key a decode reads, once per KV head
                  (2 * L * Hkv * d * s); with a shared prefix, the prefix once.
    prefill_flops: 4 * H * d per visible (query row, key) pair; query i of a
                   sequence with context c sees c + i + 1 keys (causal).
    """
    q = np.asarray(query_lens, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    P = int(common_prefix_len)
    row_bytes = 2 * num_kv_heads * head_size * elem_bytes
    dec = q == 1
    dec_tokens = int(L[dec].sum())
    if P:
        dec_tokens_read = P + int((L[dec] - P).sum())
    else:
        dec_tokens_read = dec_tokens
    ctx = L - q
    if causal:
        visible = int(np.sum(q[~dec] * ctx[~dec] + q[~dec] * (q[~dec] + 1) // 2))
    else:
        visible = int(np.sum(q[~dec] * L[~dec]))
    flops_per_pair = 4 * num_heads * head_size
    return {
        "decode_seqs": int(dec.sum()),
        "decode_kv_tokens": dec_tokens,
        "decode_bytes": dec_tokens_read * row_bytes,
        "decode_bytes_naive": dec_tokens * row_bytes,
        "decode_flops": 4 * num_heads * head_size * dec_tokens,
        "prefill_tokens": int(q[~dec].sum()),
        "prefill_pairs": visible,
        "prefill_flops": visible * flops_per_pair,
        "prefill_kv_bytes": int(L[~dec].sum()) * row_bytes,
        "prefix_flops": 4 * num_heads * head_size * P * int(q.sum()) if P else 0,
    }


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def _batch_to_device(batch, common_prefix_len=None, kv_split_tokens=0):
    import attention_paged_kv_varlen_amd as pa
    cp = batch.common_prefix_len if common_prefix_len is None else common_prefix_len
    return pa.to_device(batch.q, batch.kv_cache, batch.block_table, batch.query_start_loc, batch.seq_lens,
                        num_heads=batch.num_heads, num_kv_heads=batch.num_kv_heads, head_size=batch.head_size,
                        block_size=batch.block_size, dtype=batch.dtype, scale=batch.scale, causal=batch.causal,
                        common_prefix_len=cp, kv_split_tokens=kv_split_tokens, device="cuda:0",
                        kv_dtype=batch.kv_dtype, k_scale=batch.k_scale, v_scale=batch.v_scale,
                        kv_layout=batch.kv_layout)


def time_steps(db, steps: int, warmup: int) -> dict:
    """Warm up, then time `steps` forwards: wall clock between synchronisations
    (ms_per_step) and HIP events on the caller's stream around each forward
    (the step's device time; the side stream joins it before the forward
    ends).  Then the same number of forwards again with the HIP events the
    library records around each of its launches (per kernel: average, median,
    shortest and longest launch): those records sit between the launches and
    lengthen a step of several kernels by about 20 us, so the step is timed
    without them."""
    import torch

    import attention_paged_kv_varlen_amd as pa
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        db.forward(stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        db.forward(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pa.pa_profile_start(steps * 8 + 8)
    for _ in range(steps):
        db.forward(stream)
    torch.cuda.synchronize()
    kern = pa.pa_profile_stop()
    step = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return {
        "ms_per_step": (t1 - t0) * 1e3 / steps,
        "step_event_ms": {"median": float(np.median(step)), "min": step[0], "max": step[-1]},
        "kernels": {k["name"]: {"launches": k["launches"], "avg_us": 1e3 * k["total_ms"] / max(k["launches"], 1),
                                "median_us": 1e3 * k["median_ms"], "min_us": 1e3 * k["min_ms"],
                                "max_us": 1e3 * k["max_ms"]}
                    for k in kern},
    }


def launch_stats(k) -> dict:
    """Per-launch event times of one kernel family (us)."""
    return {x: round(k[f"{x}_us"], 3) for x in ("avg", "median", "min", "max")}


def time_graph(db, steps: int, warmup: int) -> float:
    """ms per step when one forward is captured into a HIP graph
    (torch.cuda.CUDAGraph) and replayed: the launch cost of the step's kernels
    is paid once at capture."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        db.forward()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        db.forward()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def _traffic(kernel_name: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when it is missing, was taken on another workload, or the kernel source
    changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(f"{kernel_name}@{workload}")
    if not ent or ent.get("workload") != workload:
        return None
    with open(KERNEL_SRC, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if ent.get("kernel_source_sha256") != sha:
        return None
    return ent.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline (the oracle, untuned, one thread)
# ---------------------------------------------------------------------------

def _cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: model name, family, model,
    stepping, and the logical CPUs the file lists."""
    fields, n = {}, 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key = line.split(":", 1)[0].strip()
                if key == "processor":
                    n += 1
                if key in ("model name", "cpu family", "model", "stepping") and key not in fields:
                    fields[key] = line.split(":", 1)[1].strip()
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    return (f"{name} (family {fields.get('cpu family', '?')}, model {fields.get('model', '?')}, "
            f"stepping {fields.get('stepping', '?')}; {n} logical CPUs listed)")


def _blas_name() -> str:
    try:
        b = np.__config__.CONFIG["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except (AttributeError, KeyError, TypeError):
        return "unknown"


def copy_gbs(nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Bandwidth of a plain device-to-device copy of `nbytes` on this machine (bytes
    read plus bytes written per second, best of `reps` event-timed copies): the
    copy-kernel figure reported beside the spec peak."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del src, dst
    return 2 * nbytes / best / 1e9


def sustained_mfma() -> dict | None:
    """The chip's sustained bf16 MFMA rate on random operands, bare and with
    the softmax's per-score VALU work interleaved, and the clock it settles at
    (attention_paged_kv_varlen_amd/chip_probe --json, run as a child process,
    about 0.2 s of GPU time): the measured figure reported beside the spec
    peak of MFMA-bound lines.  None when the probe is not built or fails."""
    import subprocess
    exe = os.path.join(ROOT, "attention_paged_kv_varlen_amd", "chip_probe")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe, "--json"], capture_output=True, text=True, timeout=60)
        return json.loads(r.stdout.strip().splitlines()[-1]) if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError, ValueError, IndexError):
        return None


def hbm_read_probe() -> dict | None:
    """The chip's streaming HBM read rate: a 4 GiB buffer read once per launch
    with 16-byte loads, best of plain / non-temporal loads and 2 / 4 / 8
    workgroups per CU (attention_paged_kv_varlen_amd/chip_probe --read-json,
    run as a child process, about 0.1 s of GPU time): the measured ceiling
    reported beside the spec peak of HBM-bound lines.  None when the probe is
    not built or fails."""
    import subprocess
    exe = os.path.join(ROOT, "attention_paged_kv_varlen_amd", "chip_probe")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe, "--read-json"], capture_output=True, text=True, timeout=60)
        return json.loads(r.stdout.strip().splitlines()[-1]) if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError, ValueError, IndexError):
        return None


def cpu_threads() -> int:
    """Host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def cpu_baseline(batch, counts, budget_s: float = 8.0, repeats: int = 3) -> dict:
    """Time the oracle on a bounded sample of the same batch, with BLAS threads
    set to the host cores this process may use: whole sequences in a fixed
    random order until `budget_s` of oracle time (the sample), then the same
    sample again `repeats - 1` times; the best of the repeats counts."""
    from threadpoolctl import threadpool_limits

    import oracle
    threads = cpu_threads()
    rng = np.random.default_rng(0)
    order = rng.permutation(batch.num_seqs)
    qsl = batch.query_start_loc
    L = batch.seq_lens.astype(np.int64)
    ql = np.diff(qsl).astype(np.int64)
    elem = 1 if batch.kv_dtype == "fp8_e4m3" else (2 if batch.dtype == "bf16" else 4)
    row_bytes = 2 * batch.num_kv_heads * batch.head_size * elem

    def run(b):
        oracle.attention_rows(batch.q, batch.kv_cache, batch.block_table, qsl, batch.seq_lens, batch.scale,
                              np.arange(qsl[b], qsl[b + 1]), dtype=batch.dtype, causal=batch.causal,
                              kv_dtype=batch.kv_dtype, k_scale=1.0 if batch.k_scale is None else batch.k_scale,
                              v_scale=1.0 if batch.v_scale is None else batch.v_scale)

    sample, times = [], []
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        for b in order:
            run(b)
            sample.append(int(b))
            if time.perf_counter() - t0 >= budget_s:
                break
        times.append(time.perf_counter() - t0)
        for _ in range(repeats - 1):
            t0 = time.perf_counter()
            for b in sample:
                run(b)
            times.append(time.perf_counter() - t0)
    best = min(times)
    done_bytes = sum(int(L[b]) * row_bytes for b in sample if ql[b] == 1)
    done_flops = sum(4 * batch.num_heads * batch.head_size * int(ql[b] * (L[b] - ql[b]) + ql[b] * (ql[b] + 1) // 2)
                     for b in sample if ql[b] != 1)
    res = {"cores": threads, "kind": "oracle", "seconds": round(best, 3),
           "seconds_each_repeat": [round(x, 3) for x in times],
           "sample": f"{len(sample)} of {batch.num_seqs} sequences of the same batch (numpy float64, "
                     f"BLAS threads = {threads} host cores; best of {len(times)})",
           "cpu_model": _cpu_model(), "blas": _blas_name()}
    if counts["decode_seqs"] and done_bytes:
        res.update(value=done_bytes / best / 1e9, unit="GB/s")
    else:
        res.update(value=done_flops / best / 1e12, unit="TFLOP/s")
    return res


# ---------------------------------------------------------------------------

def measure(cfg: int, steps: int, warmup: int, seed=None, kv_dtype: str = "same", kv_layout: str = "NHD",
            block_size=None) -> dict:
    """Generate the workload, time it, and return the measurement record."""
    import attention_paged_kv_varlen_amd as pa
    from workloads import config_batch
    batch = config_batch(cfg, seed=seed, kv_dtype=kv_dtype, kv_layout=kv_layout, block_size=block_size)
    s = 1 if kv_dtype == "fp8_e4m3" else (2 if batch.dtype == "bf16" else 4)
    counts = algorithmic_counts(batch.query_lens, batch.seq_lens, num_heads=batch.num_heads,
                                num_kv_heads=batch.num_kv_heads, head_size=batch.head_size, elem_bytes=s,
                                common_prefix_len=batch.common_prefix_len, causal=batch.causal)
    db = _batch_to_device(batch)
    info = pa.pa_plan_get_info(db.plan)
    t = time_steps(db, steps, warmup)
    return {"cfg": cfg, "batch": batch, "counts": counts, "timing": t, "plan": info, "db": db}


def measure_sub_plans(m, steps: int, warmup: int) -> dict:
    """The decode part and the prefill part of a mixed batch, each run as a plan
    of its own over the same device pool: decode GB/s and prefill TFLOP/s
    without the other part beside them."""
    import attention_paged_kv_varlen_amd as pa
    batch, db = m["batch"], m["db"]
    qsl = batch.query_start_loc
    ql = np.diff(qsl)
    elem = 1 if batch.kv_dtype == "fp8_e4m3" else (2 if batch.dtype == "bf16" else 4)
    res = {}
    for tag, idx in (("decode_only", np.where(ql == 1)[0]), ("prefill_only", np.where(ql != 1)[0])):
        if len(idx) == 0:
            continue
        rows = np.concatenate([np.arange(qsl[b], qsl[b + 1]) for b in idx])
        sub_qsl = np.concatenate([[0], np.cumsum(ql[idx])]).astype(np.int32)
        sub_L = np.ascontiguousarray(batch.seq_lens[idx])
        sdb = pa.to_device(np.ascontiguousarray(batch.q[rows]), batch.kv_cache,
                           np.ascontiguousarray(batch.block_table[idx]), sub_qsl, sub_L,
                           num_heads=batch.num_heads, num_kv_heads=batch.num_kv_heads, head_size=batch.head_size,
                           block_size=batch.block_size, dtype=batch.dtype, scale=batch.scale, causal=batch.causal,
                           device="cuda:0", kv_cache_dev=db.kv_cache, kv_dtype=batch.kv_dtype,
                           k_scale=batch.k_scale, v_scale=batch.v_scale, kv_layout=batch.kv_layout)
        c = algorithmic_counts(ql[idx], sub_L, num_heads=batch.num_heads, num_kv_heads=batch.num_kv_heads,
                               head_size=batch.head_size, elem_bytes=elem, causal=batch.causal)
        t = time_steps(sdb, steps, warmup)
        ms = t["ms_per_step"]
        ent = {"ms_per_step": round(ms, 5), "kernels_us": {k: round(v["avg_us"], 3) for k, v in t["kernels"].items()}}
        if tag == "decode_only":
            _, k = _kernel(t, "decode_")
            ent.update(value=round(c["decode_bytes"] / (ms * 1e-3) / 1e9, 2), unit="GB/s",
                       kernel_GBps=round(c["decode_bytes"] / (k["avg_us"] * 1e-6) / 1e9, 2))
        else:
            _, k = _kernel(t, "prefill_")
            ent.update(value=round(c["prefill_flops"] / (ms * 1e-3) / 1e12, 2), unit="TFLOP/s",
                       kernel_TFLOPs=round(c["prefill_flops"] / (k["avg_us"] * 1e-6) / 1e12, 2))
        res[tag] = ent
        del sdb
    return res


def _kernel(t, prefix):
    for name, k in t["kernels"].items():
        if name.startswith(prefix):
            return name, k
    return None, None


def summarize_pmc(fetch_csv: str, write_csv: str, copy_bytes: int, command: str, workload: str,
                  kernels=("prefix_decode_kernel", "decode_kernel", "prefill_wide_kernel", "merge_kernel")) -> dict:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) of `bench.py --workload <workload>` into HBM bytes per launch of
    each kernel, each counter scaled by what it reads for the plain device copy
    of `copy_bytes` bytes in the same run, and write them to
    profiles/traffic_counters.json."""
    import csv

    def per_dispatch(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            vals.setdefault((row["Kernel_Name"], row["Dispatch_Id"]), 0.0)
            vals[(row["Kernel_Name"], row["Dispatch_Id"])] += float(row["Counter_Value"])
        out = {}
        for (name, _), v in vals.items():
            out.setdefault(name, []).append(v)
        return out

    fd = per_dispatch(fetch_csv, "FETCH_SIZE")
    wd = per_dispatch(write_csv, "WRITE_SIZE")
    fetch = {k: sum(v) / len(v) for k, v in fd.items()}
    write = {k: sum(v) / len(v) for k, v in wd.items()}
    # the calibration copy is the largest copy dispatch (small host uploads use
    # the same copy kernel)
    copy_f = [x for k, v in fd.items() if "copy" in k.lower() for x in v]
    copy_w = [x for k, v in wd.items() if "copy" in k.lower() for x in v]
    f_scale = copy_bytes / (max(copy_f) * 1024.0)
    w_scale = copy_bytes / (max(copy_w) * 1024.0)
    with open(KERNEL_SRC, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    try:
        with open(TRAFFIC_FILE) as f:
            res = json.load(f)
    except (OSError, ValueError):
        res = {}
    calib = {"copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale, "command": command}
    res["_calibration"] = calib
    families = {"prefix_decode_kernel": "prefix_decode", "decode_kernel": "decode", "prefill_wide_kernel": "prefill",
                "merge_kernel": "merge"}
    for name in fetch:
        # the longest family name that the kernel's name holds (prefix_decode_kernel holds decode_kernel)
        fam = max((k for k in kernels if k in name), key=len, default=None)
        if fam is None or name not in write:
            continue
        family = families[fam]
        tag = ("bf16_e4m3_d128" if "unsigned char, 128" in name else
               "bf16_d128" if "unsigned short, 128" in name or "prefill_wide" in name or fam == "prefix_decode_kernel"
               else None)
        if tag is None:
            continue
        fb = fetch[name] * 1024.0 * f_scale
        wb = write[name] * 1024.0 * w_scale
        res[f"{family}_{tag}@{workload}"] = {"kernel": name, "workload": workload, "fetch_bytes_per_launch": fb,
                                  "write_bytes_per_launch": wb, "bytes_per_launch": fb + wb,
                                  "kernel_source_sha256": sha, "calibration": calib}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(res, f, indent=1)
    return res


def kvwrite_line(steps: int, warmup: int, cpu: bool, kv_dtype: str = "same") -> dict:
    """The cache write on its own: every token of the causal varlen prefill batch
    (a fresh K and V row each) written to its slot.  HBM-bound: each row is read
    once and written once (into an e4m3 pool: bf16 rows read, one-byte codes
    written, with per-head K/V scales)."""
    import torch

    import attention_paged_kv_varlen_amd as pa
    from workloads import config_batch, f32_to_bf16_bits
    batch = config_batch(3, poison=False)
    T, Hkv, d, bs = batch.num_tokens, batch.num_kv_heads, batch.head_size, batch.block_size
    qsl, L, bt = batch.query_start_loc, batch.seq_lens, batch.block_table
    # the caller's slot mapping: query token i of sequence b is key position c_b + i
    slots = np.empty(T, dtype=np.int64)
    for b in range(batch.num_seqs):
        q0, q1 = int(qsl[b]), int(qsl[b + 1])
        pos = int(L[b]) - (q1 - q0) + np.arange(q1 - q0)
        slots[q0:q1] = bt[b, pos // bs].astype(np.int64) * bs + pos % bs
    rng = np.random.default_rng(30)
    k = f32_to_bf16_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32))
    dev = "cuda:0"
    tk = torch.from_numpy(k).view(torch.bfloat16).to(dev)
    tv = torch.from_numpy(v).view(torch.bfloat16).to(dev)
    ts = torch.from_numpy(slots).to(dev)
    f8 = kv_dtype == "fp8_e4m3"
    params = pa.make_params(num_seqs=batch.num_seqs, num_heads=batch.num_heads, num_kv_heads=Hkv, head_size=d,
                            block_size=bs, num_blocks=batch.num_blocks, max_blocks_per_seq=batch.max_blocks_per_seq,
                            dtype="bf16", scale=batch.scale, kv_dtype=kv_dtype)
    if f8:
        pool = torch.zeros(batch.kv_cache.shape, dtype=torch.uint8, device=dev)
        ksc = torch.from_numpy(rng.uniform(0.005, 0.007, size=Hkv).astype(np.float32)).to(dev)
        vsc = torch.from_numpy(rng.uniform(0.005, 0.007, size=Hkv).astype(np.float32)).to(dev)
        write = lambda st: pa.pa_write_kv_fp8(tk, tv, ts, T, params, ksc, vsc, pool, stream=st)  # noqa: E731
        kname = "write_kv_e4m3"
    else:
        pool = torch.from_numpy(batch.kv_cache).view(torch.bfloat16).to(dev)
        write = lambda st: pa.pa_write_kv(tk, tv, ts, T, params, pool, st)  # noqa: E731
        kname = "write_kv"
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        write(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        write(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # per-launch events in a pass of their own (they are not part of the step)
    pa.pa_profile_start(steps + 8)
    for _ in range(steps):
        write(stream)
    torch.cuda.synchronize()
    kern = pa.pa_profile_stop()
    us = {x["name"]: 1e3 * x["total_ms"] / max(x["launches"], 1) for x in kern}
    # K and V rows read once (bf16) and written once (bf16, or one-byte codes)
    nbytes = T * 2 * Hkv * d * (2 + (1 if f8 else 2))
    ach = nbytes / (us[kname] * 1e-6) / 1e9
    line = {
        "metric": "KV-cache write GB/s (% HBM peak)", "value": round(nbytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) K/V rows)",
        "config": {"workload": f"cache write of the {T} tokens of the causal varlen prefill batch "
                               f"({Hkv} kv heads, d={d}, bs={bs}, random page placement)", "num_tokens": T},
        "kernels_us": {n: round(x, 3) for n, x in us.items()},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(ach, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None},
        "algorithmic": {"bytes": nbytes},
    }
    if f8:
        line["config"]["workload"] = line["config"]["workload"].replace("cache write", "cache write into an e4m3 pool")
        line["config"]["kv_dtype"] = kv_dtype
    if cpu:
        import oracle
        n = min(T, 4096)
        t1 = time.perf_counter()
        if f8:
            from oracle import fp8 as ofp8
            def vals(bits):  # bf16 bit patterns -> their float32 values
                return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
            ofp8.write_kv_fp8(np.zeros(batch.kv_cache.shape, dtype=np.uint8), vals(k[:n]), vals(v[:n]), slots[:n],
                              ksc.cpu().numpy(), vsc.cpu().numpy())
        else:
            oracle.write_kv(batch.kv_cache, k[:n], v[:n], slots[:n])
        dt = time.perf_counter() - t1
        line["cpu_baseline"] = {"value": n * 2 * Hkv * d * (2 + (1 if f8 else 2)) / dt / 1e9, "unit": "GB/s",
                                "cores": 1, "kind": "oracle", "seconds": round(dt, 3),
                                "sample": f"{n} of {T} tokens (numpy, one pool copy included)"}
    return line


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=sorted(WORKLOADS) + ["kvwrite"], default="decode")
    ap.add_argument("--kv-layout", choices=["NHD", "HND"], default="NHD",
                    help="memory order of the pool (HND: KV head before slot)")
    ap.add_argument("--block-size", type=int, default=None, help="page size override (a multiple of 16)")
    ap.add_argument("--kv-dtype", choices=["same", "fp8_e4m3"], default=None,
                    help="element type of the pool (default: the workload's; decode_e4m3 = decode + fp8_e4m3)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured into a HIP graph and replayed (key 'graph')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the extra measurements: the prefill in the decode line, the mixed line's "
                         "sub-plans and the device-copy bandwidth")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle work in the cpu_baseline sample (timed 3 times)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_counters.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--pmc-command", default="", help="command recorded with --summarize-pmc")
    ap.add_argument("--pmc-kernels", default="prefix_decode_kernel,decode_kernel,prefill_wide_kernel,merge_kernel",
                    help="kernel families --summarize-pmc records (comma-separated)")
    ap.add_argument("--pmc-workload", default="decode",
                    help="the --workload of the profiled runs that --summarize-pmc reads (default workload "
                         "options); the counters serve only lines of that workload")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        res = summarize_pmc(*args.summarize_pmc, copy_bytes=args.copy_calibration_mib << 20,
                            command=args.pmc_command, workload=args.pmc_workload,
                            kernels=tuple(args.pmc_kernels.split(",")))
        print(json.dumps(res, indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); sharding the "
              "batch over several GPUs is not built.", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "kvwrite":
        print(json.dumps(kvwrite_line(args.steps, args.warmup, not args.no_cpu_baseline,
                                      kv_dtype=args.kv_dtype or "same")), flush=True)
        return 0
    cfg = WORKLOADS[args.workload]
    kv_dtype = args.kv_dtype or KV_DTYPES.get(args.workload, "same")
    m = measure(cfg, args.steps, args.warmup, kv_dtype=kv_dtype, kv_layout=args.kv_layout,
                block_size=args.block_size)
    batch, counts, t = m["batch"], m["counts"], m["timing"]
    ms = t["ms_per_step"]
    dtype = batch.dtype
    # counters serve only a run of the workload they were taken on, with its
    # default pool (element type, memory order, page size)
    default_pool = (kv_dtype == KV_DTYPES.get(args.workload, "same") and args.kv_layout == "NHD"
                    and args.block_size is None)
    traffic_key = args.workload if default_pool else None
    line = {
        "metric": METRIC,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, random page placement)",
        "config": {"workload": DESCRIPTIONS[cfg] if kv_dtype == "same" else
                   DESCRIPTIONS[cfg].replace("bf16,", "bf16 queries, e4m3 KV pool (per-head K/V scales),"),
                   "num_seqs": batch.num_seqs, "num_tokens": batch.num_tokens,
                   "num_heads": batch.num_heads, "num_kv_heads": batch.num_kv_heads,
                   "head_size": batch.head_size, "block_size": batch.block_size,
                   "common_prefix_len": batch.common_prefix_len, "seed": cfg,
                   "kv_split_tokens": m["plan"]["kv_split_tokens"],
                   "decode_lists": m["plan"]["num_decode_lists"],
                   "prefix_beside_decode": m["plan"]["prefix_beside_decode"],
                   "prefix_items": m["plan"]["num_prefix_items"]},
        "step_event_ms": {k: round(v, 5) for k, v in t["step_event_ms"].items()},
        "kernels_us": {k: round(v["avg_us"], 3) for k, v in t["kernels"].items()},
        "kernel_launch_us": {k: launch_stats(v) for k, v in t["kernels"].items()},
    }
    bound = "hbm"
    if counts["decode_seqs"] and not counts["prefill_tokens"]:
        value = counts["decode_bytes"] / (ms * 1e-3) / 1e9
        line.update(value=round(value, 2), unit="GB/s")
        kname, k = _kernel(t, "decode_")
        ach = counts["decode_bytes"] / (k["avg_us"] * 1e-6) / 1e9 if k else 0.0
        if cfg == 5:
            fused, kf = _kernel(t, "prefix_decode_")
            if kf:  # the prefix pass and the decode in one launch: all the cascade's bytes
                kname, k = fused, kf
                ach = counts["decode_bytes"] / (k["avg_us"] * 1e-6) / 1e9
            else:  # the decode kernel reads only the suffixes
                elem = 1 if kv_dtype == "fp8_e4m3" else (2 if dtype == "bf16" else 4)
                suffix = counts["decode_bytes"] - batch.common_prefix_len * 2 * batch.num_kv_heads * batch.head_size * elem
                ach = suffix / (k["avg_us"] * 1e-6) / 1e9
            line["cascade"] = {"effective_GBps_vs_naive_bytes": round(counts["decode_bytes_naive"] / (ms * 1e-3) / 1e9, 1),
                               "naive_bytes": counts["decode_bytes_naive"], "cascade_bytes": counts["decode_bytes"]}
        roof = {"bound": bound, "kernel": kname, "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "launch_us": launch_stats(k)}
        roof["traffic"] = _traffic(kname, traffic_key)
    elif counts["prefill_tokens"] and not counts["decode_seqs"]:
        bound = "mfma"
        value = counts["prefill_flops"] / (ms * 1e-3) / 1e12
        line.update(value=round(value, 2), unit="TFLOP/s")
        kname, k = _kernel(t, "prefill_")
        ach = counts["prefill_flops"] / (k["avg_us"] * 1e-6) / 1e12
        peak = MFMA_PEAK_TFLOPS[dtype]
        roof = {"bound": bound, "kernel": kname, "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "launch_us": launch_stats(k), "traffic": _traffic(kname, traffic_key)}
    else:
        # mixed step: the roofline of the whole step is max(bytes/BW, flops/peak)
        peak = MFMA_PEAK_TFLOPS[dtype]
        t_ideal = max(counts["decode_bytes"] / (HBM_PEAK_GBS * 1e9), counts["prefill_flops"] / (peak * 1e12))
        value = t_ideal / (ms * 1e-3) * 100.0
        line.update(value=round(value, 2), unit="% of step roofline max(bytes/HBM, flops/MFMA)")
        kd, d = _kernel(t, "decode_")
        kp, p = _kernel(t, "prefill_")
        dec_ach = counts["decode_bytes"] / (d["avg_us"] * 1e-6) / 1e9 if d else 0.0
        pre_ach = counts["prefill_flops"] / (p["avg_us"] * 1e-6) / 1e12 if p else 0.0
        roof = {"bound": "hbm", "kernel": kd, "achieved": round(dec_ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dec_ach / HBM_PEAK_GBS, 4), "launch_us": launch_stats(d) if d else None,
                "traffic": _traffic(kd, traffic_key),
                "prefill": {"kernel": kp, "achieved_TFLOPs": round(pre_ach, 2), "peak": peak,
                            "frac": round(pre_ach / peak, 4), "launch_us": launch_stats(p) if p else None}}
        line["decode_GBps_step"] = round(counts["decode_bytes"] / (ms * 1e-3) / 1e9, 2)
        line["prefill_TFLOPs_step"] = round(counts["prefill_flops"] / (ms * 1e-3) / 1e12, 2)
    # extra measurements (left out of profiled runs with --no-secondary, so that
    # a kernel trace holds only the step's own launches)
    if roof["bound"] == "hbm" and not args.no_secondary:
        roof["copy_kernel_GBps"] = round(copy_gbs(), 1)
        rp = hbm_read_probe()
        if rp:
            roof["hbm_read_probe"] = rp
            roof["frac_of_measured_read"] = round(roof["achieved"] / rp["hbm_read_GBps"], 4)
    if roof["bound"] == "mfma" and dtype == "bf16" and not args.no_secondary:
        sm = sustained_mfma()
        if sm:
            roof["sustained_mfma"] = sm
            roof["frac_of_sustained_softmax_mix"] = round(roof["achieved"] / sm["mfma_bf16_softmax_valu_TFLOPs"], 4)
    line["roofline"] = roof
    if counts["decode_seqs"] and counts["prefill_tokens"] and not args.no_secondary:
        line["sub_plans"] = measure_sub_plans(m, args.steps, args.warmup)
    if args.graph:
        gms = time_graph(m["db"], args.steps, args.warmup)
        line["graph"] = {"ms_per_step": round(gms, 5), "value": round(line["value"] * ms / gms, 2),
                         "unit": line["unit"]}
    line["algorithmic"] = {k: counts[k] for k in ("decode_bytes", "prefill_flops", "decode_kv_tokens",
                                                  "prefill_tokens")}

    if args.kv_layout != "NHD" or args.block_size is not None:
        line["config"]["kv_layout"] = args.kv_layout
        line["config"]["block_size"] = batch.block_size
        line["config"]["workload"] += f" [pool {args.kv_layout}, bs={batch.block_size}]"
    if kv_dtype != "same":
        line["config"]["kv_dtype"] = kv_dtype
        line["data"] = "synthetic (seeded N(0,1) Q; random e4m3 codes and per-head scales; random page placement)"
    if args.workload == "decode" and not args.no_secondary:
        del m
        p = measure(3, args.steps, args.warmup)
        kp, k = _kernel(p["timing"], "prefill_")
        pf = p["counts"]["prefill_flops"]
        line["secondary"] = {
            "workload": DESCRIPTIONS[3],
            "ms_per_step": round(p["timing"]["ms_per_step"], 5),
            "step_event_ms": {x: round(v, 5) for x, v in p["timing"]["step_event_ms"].items()},
            "value": round(pf / (p["timing"]["ms_per_step"] * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "kernel": kp, "achieved": round(pf / (k["avg_us"] * 1e-6) / 1e12, 2),
                         "peak": MFMA_PEAK_TFLOPS["bf16"],
                         "frac": round(pf / (k["avg_us"] * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
                         "launch_us": launch_stats(k),
                         "frac_at_median_launch": round(pf / (k["median_us"] * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
                         "traffic": _traffic(kp, "prefill")},
        }
        sm = sustained_mfma()
        if sm:
            rf = line["secondary"]["roofline"]
            rf["sustained_mfma"] = sm
            rf["frac_of_sustained_softmax_mix"] = round(rf["achieved"] / sm["mfma_bf16_softmax_valu_TFLOPs"], 4)
        del p
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(batch, counts, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
