"""Host-side logic of bench.py (no GPU): the HBM-traffic summary from two
rocprofv3 counter runs, which lines may use it, and the one-GPU exit."""
import csv
import json

import pytest

import bench

DEC = "void pa::(anonymous namespace)::decode_kernel<unsigned short, unsigned short, 128>(pa::(anonymous namespace)::KArgs)"
MRG = "void pa::(anonymous namespace)::merge_kernel<unsigned short, 128>(pa::MergeRow const*, int)"
COPY = "__amd_rocclr_copyBuffer"


def _counter_csv(path, counter, rows):
    # rows: (kernel, dispatch, KiB); a dispatch may report several partial values (per XCD)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, d, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


@pytest.fixture
def traffic_file(tmp_path, monkeypatch):
    p = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    return p


def test_summary_scales_by_the_largest_copy_and_binds_the_workload(tmp_path, traffic_file):
    mib = 1 << 20
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the 1 GiB copy reads as 2 x its size in FETCH_SIZE (KiB) and 1 x in WRITE_SIZE;
    # a small host upload through the same copy kernel must not set the scale
    _counter_csv(fetch, "FETCH_SIZE", [(COPY, 1, 2 * 1024 * 1024), (COPY, 2, 10),
                                       (DEC, 3, 300.0), (DEC, 3, 100.0), (DEC, 4, 500.0),
                                       (MRG, 5, 8.0)])
    _counter_csv(write, "WRITE_SIZE", [(COPY, 1, 1024 * 1024), (COPY, 2, 999),
                                       (DEC, 3, 20.0), (DEC, 4, 20.0), (MRG, 5, 4.0)])
    res = bench.summarize_pmc(str(fetch), str(write), copy_bytes=1024 * mib, command="cmd", workload="decode")
    dec = res["decode_bf16_d128@decode"]
    # per dispatch: 400 and 500 KiB fetched -> 450 KiB mean, halved by the calibration
    assert dec["fetch_bytes_per_launch"] == pytest.approx(450 * 1024 / 2)
    assert dec["write_bytes_per_launch"] == pytest.approx(20 * 1024)
    assert dec["bytes_per_launch"] == pytest.approx(450 * 512 + 20 * 1024)
    assert dec["workload"] == "decode" and res["merge_bf16_d128@decode"]["workload"] == "decode"
    assert res["_calibration"]["fetch_scale"] == pytest.approx(0.5)
    assert json.loads(traffic_file.read_text())["decode_bf16_d128@decode"]["kernel"] == DEC


def test_traffic_serves_only_its_workload_and_source(tmp_path, traffic_file, monkeypatch):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fetch, "FETCH_SIZE", [(COPY, 1, 2048.0), (DEC, 2, 64.0)])
    _counter_csv(write, "WRITE_SIZE", [(COPY, 1, 1024.0), (DEC, 2, 8.0)])
    bench.summarize_pmc(str(fetch), str(write), copy_bytes=1 << 20, command="", workload="decode")
    full = bench._traffic("decode_bf16_d128", "decode")
    assert full == pytest.approx(64 * 512 + 8 * 1024)
    # another workload's line (mixed step, cascade) or a non-default pool gets none
    assert bench._traffic("decode_bf16_d128", "mixed") is None
    # counters of the same kernel on another workload sit beside, not over, these
    bench.summarize_pmc(str(fetch), str(write), copy_bytes=1 << 19, command="", workload="cascade")
    assert bench._traffic("decode_bf16_d128", "cascade") == pytest.approx(full / 2)
    assert bench._traffic("decode_bf16_d128", "decode") == pytest.approx(full)
    assert bench._traffic("decode_bf16_d128", None) is None
    assert bench._traffic("prefill_bf16_d128", "prefill") is None
    # counters taken before the kernel source changed are not used
    src = tmp_path / "kernels.hip"
    src.write_text("// changed\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    assert bench._traffic("decode_bf16_d128", "decode") is None


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_chip_probe_readers_tolerate_a_missing_or_failing_probe(tmp_path, monkeypatch):
    # no probe built: both readers return None (the bench line then leaves the
    # measured ceilings out instead of failing)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.sustained_mfma() is None and bench.hbm_read_probe() is None
    # a probe that prints JSON is parsed; one that fails is ignored
    exe = tmp_path / "attention_paged_kv_varlen_amd" / "chip_probe"
    exe.parent.mkdir()
    exe.write_text('#!/bin/sh\nif [ "$1" = "--read-json" ]; then echo \'{"hbm_read_GBps": 7000.0}\'; '
                   'else exit 3; fi\n')
    exe.chmod(0o755)
    assert bench.hbm_read_probe() == {"hbm_read_GBps": 7000.0}
    assert bench.sustained_mfma() is None
