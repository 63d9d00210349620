"""Host logic of the measurement tooling (no GPU): the traffic summary's calibration scaling and
source hashes, the per-kernel averages over the last N dispatches and over counter runs, and the
benchmark's rule of quoting a stored traffic figure only while the kernel's sources are unchanged.
The CSV files are synthetic, in the column layout rocprofv3 writes."""
import csv
import json

import pytest

import bench
from causal_gqa_flashattention_ne_amd import profsum

COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"
BWD = "void ne::(anonymous namespace)::bwd_bf16_kernel<64>(ne::BwdArgs)"
FWD = "void ne::(anonymous namespace)::fwd_bf16_kernel<64, true>(ne::FwdArgs)"


def write_counters(path, rows):
    path.mkdir(parents=True, exist_ok=True)
    with open(path / "t_counter_collection.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, counter, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_scales_by_the_copy_calibration(tmp_path):
    cal_kib = profsum.CAL_BYTES / 1024.0
    # the copy reads 256 MiB, FETCH_SIZE reports half of it; WRITE_SIZE reports all of it
    write_counters(tmp_path / "f", [(COPY, "FETCH_SIZE", cal_kib / 2), (BWD, "FETCH_SIZE", 1000.0),
                                    (BWD, "FETCH_SIZE", 3000.0)])
    write_counters(tmp_path / "w", [(COPY, "WRITE_SIZE", cal_kib), (BWD, "WRITE_SIZE", 500.0)])
    out = tmp_path / "t.json"
    profsum.traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out))
    t = json.load(open(out))
    assert t["read_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    k = t["kernels"]["bwd_main"]
    assert k["read_bytes"] == pytest.approx(2.0 * 2000.0 * 1024)        # average of the dispatches
    assert k["write_bytes"] == pytest.approx(500.0 * 1024)
    assert k["source_sha256"] == profsum.source_hash("bwd_main")


def test_traffic_needs_the_calibration_copy(tmp_path):
    write_counters(tmp_path / "f", [(BWD, "FETCH_SIZE", 1.0)])
    write_counters(tmp_path / "w", [(BWD, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        profsum.traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "t.json"))


def test_source_hash_follows_the_kernel_sources():
    # each short name hashes its own sources and the shared headers: different kernels differ,
    # the same kernel is stable
    assert profsum.source_hash("bwd_main") == profsum.source_hash("bwd_main")
    assert profsum.source_hash("bwd_main") != profsum.source_hash("decode16")
    assert len(profsum.source_hash()) == 64


def test_last_n_averages_the_latest_dispatches(tmp_path, capsys):
    p = tmp_path / "k_kernel_trace.csv"
    with open(p, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        t = 0
        for dur in (9000, 9000, 2000, 4000):          # ns, in dispatch order
            wr.writerow({"Kernel_Name": BWD, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += 10 * dur
        wr.writerow({"Kernel_Name": FWD, "Start_Timestamp": t, "End_Timestamp": t + 1000})
    profsum.last_n(2, str(p))
    lines = {l[:64].strip(): l.split() for l in capsys.readouterr().out.splitlines()[1:]}
    bwd = next(v for k, v in lines.items() if "bwd_bf16_kernel" in k)
    fwd = next(v for k, v in lines.items() if "fwd_bf16_kernel" in k)
    assert bwd[-2:] == ["2", "3.00"]                  # (2000 + 4000) / 2 ns = 3 us
    assert fwd[-2:] == ["1", "1.00"]


def test_counters_average_per_kernel(tmp_path, capsys):
    write_counters(tmp_path / "a", [(BWD, "MfmaUtil", 20.0), (BWD, "MfmaUtil", 30.0), (FWD, "MfmaUtil", 10.0)])
    write_counters(tmp_path / "b", [(BWD, "VALUBusy", 40.0)])
    profsum.counters([str(tmp_path / "a"), str(tmp_path / "b")])
    out = capsys.readouterr().out.splitlines()
    assert out[0].split()[1:] == ["MfmaUtil", "VALUBusy"]
    rows = {l.split()[0]: l.split()[1:] for l in out[1:]}
    assert rows["bwd_main"] == ["25", "40"] and rows["fwd"] == ["10", "-"]


def test_bench_quotes_traffic_only_for_unchanged_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = {"kernels": {"bwd_main": {"read_bytes": 3.0, "write_bytes": 4.0,
                                     "source_sha256": profsum.source_hash("bwd_main")}}}
    stale = {"kernels": {"bwd_main": {"read_bytes": 3.0, "write_bytes": 4.0, "source_sha256": "0" * 64}}}
    json.dump(good, open(prof / "traffic_w-good.json", "w"))
    json.dump(stale, open(prof / "traffic_w-stale.json", "w"))
    monkeypatch.setattr(bench, "__file__", str(tmp_path / "bench.py"))
    assert bench.measured_traffic("w-good", "bwd_main") == 7.0
    assert bench.measured_traffic("w-stale", "bwd_main") is None
    assert bench.measured_traffic("w-none", "bwd_main") is None
    assert bench.measured_traffic("w-good", "fwd") is None
