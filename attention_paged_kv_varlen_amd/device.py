"""Move host arrays of one batch into device tensors and run a plan on them.

Marshalling only: torch allocates device memory and provides the stream; the
attention itself runs in libpagedattn.  bf16 arrays arrive as 16-bit patterns
(``np.uint16``) and are reinterpreted as ``torch.bfloat16`` without conversion;
an e4m3 pool arrives as its 8-bit codes (``np.uint8``) and stays ``torch.uint8``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import _capi


def _to_torch(a: np.ndarray, dtype: str, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16" and t.dtype == torch.uint16:  # bf16 bit patterns (not e4m3 codes)
        t = t.view(torch.bfloat16)
    return t.to(device, non_blocking=False)


@dataclass
class DeviceBatch:
    params: _capi.pa_params
    plan: _capi.Plan
    q: object
    kv_cache: object
    block_table: object
    query_start_loc: object
    seq_lens: object
    out: object
    lse: object
    workspace: object
    k_scale: object = None  # e4m3 pool: float32 device tensors of 1 or Hkv scales
    v_scale: object = None

    def forward(self, stream=None) -> None:
        if self.k_scale is not None:
            _capi.pa_forward_fp8(self.plan, self.q, self.kv_cache, self.block_table, self.query_start_loc,
                                 self.seq_lens, self.k_scale, self.v_scale, self.out, self.lse, self.workspace,
                                 stream=stream)
        else:
            _capi.pa_forward(self.plan, self.q, self.kv_cache, self.block_table, self.query_start_loc,
                             self.seq_lens, self.out, self.lse, self.workspace, stream=stream)


def to_device(q, kv_cache, block_table, query_start_loc, seq_lens, *, num_heads, num_kv_heads, head_size,
              block_size, dtype, scale, causal=True, common_prefix_len=0, kv_split_tokens=0,
              device="cuda", kv_cache_dev=None, kv_dtype="same", k_scale=None, v_scale=None,
              kv_layout="NHD", check_metadata=False) -> DeviceBatch:
    """Build the plan and the device tensors (q, pool, table, query_start_loc,
    seq_lens, out, lse, workspace; the K/V scales of an e4m3 pool)."""
    import torch
    dev = torch.device(device)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    params = _capi.make_params(
        num_seqs=len(seq_lens), num_heads=num_heads, num_kv_heads=num_kv_heads, head_size=head_size,
        block_size=block_size, num_blocks=kv_cache.shape[0], max_blocks_per_seq=bt.shape[1], dtype=dtype,
        scale=scale, causal=causal, common_prefix_len=common_prefix_len, kv_split_tokens=kv_split_tokens,
        kv_dtype=kv_dtype, kv_layout=kv_layout, check_metadata=check_metadata)
    plan = _capi.pa_plan_create(params, query_start_loc, seq_lens, bt, device=dev.index or 0)
    tq = _to_torch(q, dtype, dev)
    tkv = kv_cache_dev if kv_cache_dev is not None else _to_torch(kv_cache, dtype, dev)
    tbt = torch.from_numpy(bt).to(dev)
    tqsl = torch.from_numpy(np.ascontiguousarray(query_start_loc, dtype=np.int32)).to(dev)
    tsl = torch.from_numpy(np.ascontiguousarray(seq_lens, dtype=np.int32)).to(dev)
    out = torch.empty_like(tq)
    lse = torch.empty(tq.shape[0], num_heads, dtype=torch.float32, device=dev)
    nws = _capi.pa_plan_workspace_bytes(plan)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    ks = vs = None
    if kv_dtype == "fp8_e4m3":
        ks = torch.from_numpy(np.ascontiguousarray(k_scale, dtype=np.float32).reshape(-1)).to(dev)
        vs = torch.from_numpy(np.ascontiguousarray(v_scale, dtype=np.float32).reshape(-1)).to(dev)
    return DeviceBatch(params, plan, tq, tkv, tbt, tqsl, tsl, out, lse, ws, ks, vs)
