"""Host-side logic of bench.py (no GPU): the counted pair number, kernel-name
parsing, and the traffic summary written from two rocprofv3 counter runs and
read back for the roofline line."""
import csv
import importlib.util
import os

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture()
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_unmasked_pairs_match_the_mask(bench):
    """U is the number of (query, key) pairs the mask allows, per head."""
    class W:
        N = 50
    for cu in (None, np.array([0, 7, 8, 30, 50])):
        i, j = np.meshgrid(np.arange(W.N), np.arange(W.N), indexing="ij")
        allowed = j <= i
        if cu is not None:
            doc = np.searchsorted(cu, np.arange(W.N), side="right") - 1
            allowed &= doc[:, None] == doc[None, :]
        assert bench.unmasked_pairs(W, cu) == int(allowed.sum())


def test_short_kernel_name(bench):
    full = "void uly::(anonymous namespace)::attn_fwd_kernel<128, 4, 2, false>(uly::(anonymous namespace)::FwdArgs)"
    assert bench.short_kernel_name(full) == "attn_fwd_kernel<128, 4, 2, false>"


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for disp, name, value in rows:
            wr.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_calibrates_on_the_pack_and_tracks_the_sources(bench, tmp_path, monkeypatch):
    """The pack reads and writes the shard's bytes exactly once, so its
    counter readings fix the two scale factors; every other dispatch is
    scaled by them. The summary stops being used once a source changes."""
    root = tmp_path / "root"
    (root / "profiles").mkdir(parents=True)
    (root / "long_context_attention_ulysses_amd" / "csrc").mkdir(parents=True)
    (root / "long_context_attention_ulysses_amd" / "csrc" / "k.hip").write_text("// v1\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    w = workloads.WORKLOADS["64k"]
    shard = w.n * w.Ht * w.d * 2
    pack = "void uly::(anonymous namespace)::swap_kernel<true>(uly::(anonymous namespace)::SwapArgs)"
    dkdv = "void uly::(anonymous namespace)::attn_bwd_dkdv_kernel<128, false>(uly::(anonymous namespace)::BwdArgs)"
    # counters in KiB; FETCH_SIZE reads half the true bytes on the pack, WRITE_SIZE all of them
    pmc = tmp_path / "pmc"
    pmc.mkdir()
    _write_counters(pmc / "fetch_counter_collection.csv", "FETCH_SIZE", [(1, pack, shard / 2 / 1024), (2, dkdv, 1000.0)])
    _write_counters(pmc / "write_counter_collection.csv", "WRITE_SIZE", [(1, pack, shard / 1024), (2, dkdv, 300.0)])
    # the clock pass: GRBM_GUI_ACTIVE summed over 8 XCDs, with the kernel trace of the same run
    _write_counters(pmc / "grbm_counter_collection.csv", "GRBM_GUI_ACTIVE",
                    [(1, pack, 8 * 2.0 * 50_000), (2, dkdv, 8 * 1.9 * 17_000_000)])
    with open(pmc / "grbm_kernel_trace.csv", "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        wr.writerow({"Dispatch_Id": 1, "Kernel_Name": pack, "Start_Timestamp": 1000, "End_Timestamp": 51_000})
        wr.writerow({"Dispatch_Id": 2, "Kernel_Name": dkdv, "Start_Timestamp": 60_000, "End_Timestamp": 17_060_000})
    bench.write_traffic_summary("64k", str(pmc))
    got = bench.measured_profile("64k", "a8_attn_bwd_dkdv")
    assert got["hbm_bytes"] == int(round((1000.0 * 2.0 + 300.0 * 1.0) * 1024))
    assert abs(got["clock_ghz"] - 1.9) < 1e-9
    assert bench.measured_profile("64k", "a3_attn_fwd") is None          # no such dispatch
    (root / "long_context_attention_ulysses_amd" / "csrc" / "k.hip").write_text("// v2\n")
    assert bench.measured_profile("64k", "a8_attn_bwd_dkdv") is None     # kernels changed since


def test_bench_refuses_more_than_one_gpu(bench, monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
