"""Host logic of bench.py (CPU only): the algorithmic byte and FLOP counts
behind the rooflines, the counter summary that scales rocprofv3 FETCH_SIZE /
WRITE_SIZE by a copy of known size, and the rule that a measured traffic
figure is reported only for the kernel source it was taken on."""
import csv
import json
import os

import pytest

import bench


def test_long_prefill_bytes_and_flops():
    # q and k once per key head, v and y, g and beta, the f32 state read and
    # written once: 2*8*8192*16*128*2 + 2*8*8192*32*128*2 + 2*8*8192*32*4
    # + 2*8*32*128*128*4, added up by hand
    assert bench.prefill_bytes(**bench.PREFILL) == 1_660_944_384
    # 6 Dk Dv + 2 C Dk + 2 C Dv = 98304 + 16384 + 16384 = 2^17 per token and
    # value head, over 8 * 8192 tokens and 32 value heads
    assert bench.prefill_flops(**bench.PREFILL) == 2 ** 17 * 8 * 8192 * 32 == 274_877_906_944


def test_decode_step_bytes():
    state, total = bench.step_bytes(**bench.DECODE)
    assert state == 2 * 64 * 32 * 128 * 128 * 4 == 268_435_456
    # plus q, k (per key head) and v, y (per value head) in f16, g and beta
    assert total == state + 524_288 + 1_048_576 + 16_384 == 270_024_704


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value})


def test_summarize_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    chunk = "_ZN3gdn15chunk_wy_kernelIDF16bLi4EEEvPKT_"
    copy = "__amd_rocclr_copyBuffer"
    # the chunk kernel's counters vary per dispatch; the mean is used.  A
    # 1 GiB copy whose FETCH_SIZE reads half its bytes gives the factor 2.
    _write_counters(tmp_path / "f", [(chunk, "FETCH_SIZE", 598000.0), (chunk, "FETCH_SIZE", 602000.0),
                                     ("other_kernel", "FETCH_SIZE", 1.0)])
    _write_counters(tmp_path / "w", [(chunk, "WRITE_SIZE", 540000.0), (chunk, "WRITE_SIZE", 540000.0)])
    _write_counters(tmp_path / "cf", [(copy, "FETCH_SIZE", 524288.0)])
    _write_counters(tmp_path / "cw", [(copy, "WRITE_SIZE", 1048576.0)])
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                            str(tmp_path / "cw"))
    rec = json.loads(out.read_text())
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["read_bytes_per_launch"] == pytest.approx(600000.0 * 2 * 1024)
    assert rec["write_bytes_per_launch"] == pytest.approx(540000.0 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx((1200000.0 + 540000.0) * 1024)
    assert rec["algorithmic_bytes_per_launch"] == 1_660_944_384
    assert rec["source_hash"] == bench.chunk_source_hash()


def test_traffic_reported_only_for_its_source(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.load_traffic() is None                      # no summary yet
    path.write_text(json.dumps({"source_hash": bench.chunk_source_hash(), "bytes_per_launch": 1.5e9}))
    assert bench.load_traffic() == 1.5e9
    path.write_text(json.dumps({"source_hash": "0" * 16, "bytes_per_launch": 1.5e9}))
    assert bench.load_traffic() is None                      # taken on another source


def test_committed_traffic_matches_the_present_source():
    """The summary under profiles/ was taken on the chunk kernel source as
    it stands, so the bench reports its traffic figure."""
    with open(os.path.join(bench.ROOT, "profiles", "chunk_long_prefill_hbm_traffic.json")) as f:
        rec = json.load(f)
    assert rec["source_hash"] == bench.chunk_source_hash()
    assert rec["algorithmic_bytes_per_launch"] == bench.prefill_bytes(**bench.PREFILL)
