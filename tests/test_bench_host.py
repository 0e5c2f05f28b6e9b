"""Host logic of bench.py that turns profiler output into the reported
figures: the kernel-trace summary (averages over exactly the timed steps)
and the HBM-traffic summary (counter values scaled by a copy of known
size).  Synthetic rocprofv3-style CSV files; no GPU."""
import csv
import json
import os

import numpy as np
import pytest

import workloads as W

import bench

PRODUCER = "void spa::(anonymous namespace)::decode_kernel<0, 2, false, true>(spa::DecodeParams)"
MERGE = "spa::(anonymous namespace)::split_merge_kernel(float const*, float const*)"
META = "spa::(anonymous namespace)::build_metadata_kernel(spa::MetadataParams)"


def _write_trace(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_trace_picks_the_timed_steps(tmp_path):
    # dispatch order of a bench run: the rig's first metadata build, then W
    # warm-up steps, K timed steps and K evented steps of (meta, producer, merge)
    W, K = 3, 4
    rows, t = [], 0
    # durations encode the phase: warm-up 100 us, timed 200, evented 300
    def add(name, us):
        nonlocal t
        rows.append({"Kernel_Name": name, "Start_Timestamp": t,
                     "End_Timestamp": t + int(us * 1000)})
        t += int(us * 1000) + 10
    add(META, 1.0)
    for phase, us in (("warm", 100.0), ("timed", 200.0), ("evented", 300.0)):
        for _ in range(W if phase == "warm" else K):
            add(META, us / 100)
            add(PRODUCER, us)
            add(MERGE, us / 50)
    rows = rows[::-1]                      # file order must not matter
    _write_trace(tmp_path / "run_kernel_trace.csv", rows)
    s = bench.summarize_trace(str(tmp_path), W, K)
    assert s["producer"]["timed_steps_avg_us"] == pytest.approx(200.0)
    assert s["producer"]["event_steps_avg_us"] == pytest.approx(300.0)
    assert s["split_merge"]["timed_steps_avg_us"] == pytest.approx(4.0)
    assert s["metadata"]["timed_steps_avg_us"] == pytest.approx(2.0)
    assert s["metadata"]["event_steps_avg_us"] == pytest.approx(3.0)
    assert s["producer"]["dispatches"] == W + 2 * K
    assert s["metadata"]["dispatches"] == 1 + W + 2 * K
    n = W + 2 * K
    assert s["producer"]["all_avg_us"] == pytest.approx((100 * W + 200 * K + 300 * K) / n)


def _write_pmc(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_pmc_scales_by_the_copy(tmp_path, monkeypatch):
    # the fetch counter reads half of what a 1 MiB copy moves; write reads it
    # all; values arrive split over dimension rows of one dispatch
    fdir, wdir = tmp_path / "f", tmp_path / "w"
    fdir.mkdir()
    wdir.mkdir()
    copy_kib = 1024
    f_rows = [
        {"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": copy_kib / 2 / 2},
        {"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": copy_kib / 2 / 2},
        {"Dispatch_Id": 2, "Kernel_Name": PRODUCER, "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 500.0},
        {"Dispatch_Id": 3, "Kernel_Name": MERGE, "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 10.0},
    ]
    w_rows = [
        {"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
         "Counter_Value": copy_kib},
        {"Dispatch_Id": 2, "Kernel_Name": PRODUCER, "Counter_Name": "WRITE_SIZE",
         "Counter_Value": 8.0},
        {"Dispatch_Id": 3, "Kernel_Name": MERGE, "Counter_Name": "WRITE_SIZE",
         "Counter_Value": 1.0},
    ]
    _write_pmc(fdir / "run_counter_collection.csv", "FETCH_SIZE", f_rows)
    _write_pmc(wdir / "run_counter_collection.csv", "WRITE_SIZE", w_rows)
    monkeypatch.setattr(bench, "_source_hash", lambda kind: "h")
    out = tmp_path / "traffic.json"
    rec = bench.summarize_pmc(str(fdir), str(wdir), str(out), 1, "w", ["cmd"])
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    d = rec["kernels"]["decode"]
    assert d["fetch_bytes"] == 500 * 1024 * 2 and d["write_bytes"] == 8 * 1024
    m = rec["kernels"]["split_merge"]
    assert rec["hbm_bytes_per_launch"] == d["fetch_bytes"] + d["write_bytes"] + \
        m["fetch_bytes"] + m["write_bytes"]
    assert json.load(open(out))["kernel_source_sha256"] == "h"
    # the bench reads it back only while the kernel sources are unchanged
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    os.replace(out, tmp_path / "profiles" / "traffic_w.json")
    assert bench._traffic_for("decode", "w") == rec["hbm_bytes_per_launch"]
    assert bench._traffic_for("decode", "w", producer_only=True) == \
        d["fetch_bytes"] + d["write_bytes"]
    monkeypatch.setattr(bench, "_source_hash", lambda kind: "changed")
    assert bench._traffic_for("decode", "w") is None


def test_multi_gpu_request_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err


def test_rotation_layout_copies_map_back_to_the_case_pages():
    """Each page copy's page table (the oracle's metadata definition over the
    rotated req_to_token) names, page for page, copies of the case's own
    pages; copies occupy disjoint page ranges; R copies reach 1 GiB."""
    import bench
    import oracle
    c = W.make_case(seed=3, seq_lens=[100, 7, 300, 64], num_pages=40, num_splits=4,
                    req_pool_rows=4, req_to_token_stride=1024, max_seq_pages=16,
                    num_q_heads=8, num_kv_heads=2, head_dim=16)
    R = 3
    src, r2t, rpi = W.rotation_layout(c, R)
    U = src.shape[0] // R
    assert U == sum(-(-int(L) // c.page_size) for L in c.seq_lens)
    seen = []
    for cp in range(R):
        pt, _, _ = oracle.build_page_table(r2t, rpi[cp], c.seq_lens, c.page_size,
                                           c.max_seq_pages)
        used = []
        for b in range(c.batch):
            n = -(-int(c.seq_lens[b]) // c.page_size)
            assert np.array_equal(src[pt[b, :n]], c.page_list[b, :n]), (cp, b)
            assert np.all((pt[b, :n] >= cp * U) & (pt[b, :n] < (cp + 1) * U))
            used.extend(pt[b, :n].tolist())
        assert len(set(used)) == U
        seen.extend(used)
    assert len(set(seen)) == R * U
    case4 = W.make_config(4)
    r, per = bench.rotation_copies(case4)
    assert r == 2 and r * per >= (1 << 30)
    case1_lens = W.config_seq_lens(1)
    assert bench.rotation_copies(type("C", (), dict(page_size=64, seq_lens=case1_lens,
                                                     kv_bytes_per_token=lambda s: 4096))())[0] \
        == 256
