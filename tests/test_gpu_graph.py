"""pa_forward captured into a HIP graph (torch.cuda.CUDAGraph on ROCm): every
replay, with eager work and synchronisations between replays, must give the
eager result bit for bit, including plans whose prefill or shared-prefix work
forks onto the plan's side stream."""
import numpy as np
import pytest

from tests.gpu_helpers import announce, run_gpu
from workloads import make_batch

pytestmark = pytest.mark.gpu

CASES = {
    "mixed_side_stream": dict(qlens=[1, 1, 1, 37, 130], lens=[40, 700, 2100, 337, 130]),
    "decode_only_lists": dict(qlens=[1] * 9, lens=[5, 300, 1200, 4096, 1, 77, 900, 2500, 33]),
    "cascade": dict(qlens=[1, 1, 1, 9], lens=[128 + 5, 128 + 300, 128 + 40, 128 + 9], shared_prefix_blocks=8),
    "e4m3_hnd_mixed": dict(qlens=[1, 1, 70], lens=[300, 2000, 200], kv_dtype="fp8_e4m3", kv_layout="HND"),
    # 8 KV heads, decodes alone: the prefix pass and the decode in one launch
    "cascade_fused_hkv8": dict(qlens=[1] * 6, lens=[256 + 5, 256 + 300, 256 + 40, 256 + 1, 256 + 900, 256 + 64],
                               shared_prefix_blocks=16, num_heads=32, num_kv_heads=8),
    # 8 KV heads with a prefill: prefix pass and prefill on the side stream
    "cascade_prefill_hkv8": dict(qlens=[1, 1, 1, 40], lens=[256 + 5, 256 + 300, 256 + 40, 256 + 90],
                                 shared_prefix_blocks=16, num_heads=32, num_kv_heads=8),
    # 8 KV heads, decodes and prefills (g = 8): the 8-wave prefill on the side
    # stream beside 8-wave decode workgroups
    "mixed_hkv8_g8": dict(qlens=[1, 1, 1, 1, 70, 33], lens=[40, 700, 2100, 3000, 500, 33],
                          num_heads=64, num_kv_heads=8),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    import torch
    kw = dict(CASES[name])
    qlens, lens = kw.pop("qlens"), kw.pop("lens")
    kw.setdefault("num_heads", 8)
    kw.setdefault("num_kv_heads", 2)
    b = make_batch(qlens, lens, head_size=128, block_size=16, seed=80, **kw)
    announce(f"graph {name}")
    out_e, lse_e, db = run_gpu(b)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm up on the capture stream
        db.forward()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        db.forward()
    for rep in range(3):
        db.out.zero_()
        db.lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        out = db.out.float().cpu().numpy().astype(np.float64)
        lse = db.lse.cpu().numpy().astype(np.float64)
        assert np.array_equal(out, out_e) and np.array_equal(lse, lse_e), f"replay {rep} differs"
        # eager work between replays
        db.forward()
        torch.cuda.synchronize()
        assert np.array_equal(db.out.float().cpu().numpy().astype(np.float64), out_e)
