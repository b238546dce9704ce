"""Host logic of bench.py: the algorithmic work counts and the counter bookkeeping.

No GPU: the counter files are written here with known values, in the column layout of
rocprofv3's counter_collection.csv, and the derived figures are checked by hand.
"""
import csv
import json

import numpy as np
import pytest

import bench
import workloads as W


def _brute_keys(w, seq_lens):
    """Key-set sizes counted pair by pair from the mask definition."""
    out = np.zeros((w.batch, w.q_len), np.int64)
    for b in range(w.batch):
        valid = w.kv_len if seq_lens is None else min(int(seq_lens[b]), w.kv_len)
        for i in range(w.q_len):
            p = w.pos_offset + i
            if p >= valid:
                continue
            n = 0
            for j in range(valid):
                if w.causal and j > p:
                    continue
                if w.window > 0:
                    if w.causal and j <= p - w.window:
                        continue
                    if not w.causal and abs(j - p) > w.window // 2:
                        continue
                n += 1
            out[b, i] = n
    return out


@pytest.mark.parametrize("causal,window,pos,lens", [
    (True, 0, 0, None), (False, 0, 0, [5, 40]), (False, 8, 0, None), (True, 6, 3, [30, 12]),
    (False, 8, 0, [17, 33]), (True, 0, 10, None)])
def test_keys_per_row_matches_pair_count(causal, window, pos, lens):
    w = W.Workload("t", "prefill", 2, 2, 1, 33, 40, 16, "bf16", 1.0, causal, window=window, pos_offset=pos)
    sl = None if lens is None else np.array(lens, np.int32)
    assert np.array_equal(bench.keys_per_row(w, sl), _brute_keys(w, sl))


def test_named_workload_flops():
    # causal 4096 x 4096, 32 heads, head_dim 128: 4 * 128 * 32 * 4096 * 4097 / 2
    w = W.WORKLOADS["causal_gqa_s4096"]
    assert bench.prefill_flops(w, None) == 4 * 128 * 32 * 4096 * 4097 / 2
    # band |i - j| <= 64 over 8192 keys: 8192 * 129 pairs minus the two clipped corners
    w = W.WORKLOADS["banded_w128_s8192"]
    assert bench.prefill_flops(w, None) == 4 * 64 * 12 * 8 * (8192 * 129 - 2 * (64 * 65 // 2))


def _write_counters(path, rows):
    path.mkdir(parents=True, exist_ok=True)
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path / "run_counter_collection.csv", "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=cols)
        wr.writeheader()
        for r in rows:
            wr.writerow(dict(zip(cols, r)))


def test_record_mfma(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", tmp_path / "profiles")
    (tmp_path / "profiles").mkdir()
    run = tmp_path / "runs"
    # every workload: two dispatches of 100 us and 120 us at 2.0 GHz on each XCD, MFMA busy
    # half the cycles, plus a dispatch of another kernel that must be ignored
    for name, prefix in bench.MFMA_RUNS:
        rows = []
        for d, us in ((1, 100.0), (2, 120.0)):
            cyc = 2.0e3 * us
            vals = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_BUSY_CYCLES": 1.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * cyc / 2,
                    "SQ_ACTIVE_INST_VALU": 1024 * 1000.0}
            for k, v in vals.items():
                rows.append((d, f"void mi_attn::{prefix}, 1>(args)", k, v, 0, int(us * 1e3)))
        rows.append((3, "void mi_attn::other_kernel(args)", "GRBM_GUI_ACTIVE", 1e12, 0, 10 ** 9))
        _write_counters(run / name, rows)
    out = bench.record_mfma(run)
    saved = json.loads((tmp_path / "profiles" / "mfma.json").read_text())
    for name, _ in bench.MFMA_RUNS:
        r = out[name]
        assert saved[name] == r
        assert r["dispatches"] == 2
        assert r["duration_us"] == pytest.approx(110.0)
        assert r["clock_GHz"] == pytest.approx(2.0)
        assert r["mfma_busy_frac"] == pytest.approx(0.5)
        assert r["valu_insts_per_simd"] == pytest.approx(1000.0)
        assert r["executed_mfma_flop"] == pytest.approx(1024 * 1024 * 2.0e3 * 110.0 / 2)
        w = W.WORKLOADS[name]
        sl = W.make_inputs(w)["seq_lens"] if w.seq_len_range is not None else None
        alg = bench.prefill_flops(w, sl)
        assert r["algorithmic_TFLOPs"] == pytest.approx(alg / 110e-6 / 1e12)
        assert r["frac_of_peak"] == pytest.approx(alg / 110e-6 / 1e12 / 2500.0)


def test_record_traffic(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", tmp_path / "profiles")
    (tmp_path / "profiles").mkdir()
    run = tmp_path / "runs"
    gib_kib = (1 << 30) / 1024
    # the copy reads 1 GiB and the counter shows half of it: every FETCH is scaled by 2
    _write_counters(run / "copy_FETCH_SIZE", [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2, 0, 1)])
    _write_counters(run / "copy_WRITE_SIZE", [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib, 0, 1)])
    # every workload's run holds its own kernel (two dispatches, 1000 and 3000 KiB read) and
    # a dispatch of another kernel that must be ignored
    for name, prefixes in bench.TRAFFIC_KERNELS.items():
        fetch = [(1, "void mi_attn::some_other_kernel(a)", "FETCH_SIZE", 1e9, 0, 1)]
        write = [(1, "void mi_attn::some_other_kernel(a)", "WRITE_SIZE", 1e9, 0, 1)]
        for p in prefixes:
            fetch += [(2, f"void mi_attn::{p}, 4, 1, 0>(a)", "FETCH_SIZE", 1000.0, 0, 1),
                      (3, f"void mi_attn::{p}, 4, 1, 0>(a)", "FETCH_SIZE", 3000.0, 0, 1)]
            write += [(2, f"void mi_attn::{p}, 4, 1, 0>(a)", "WRITE_SIZE", 4.0, 0, 1)]
        _write_counters(run / f"{name}_FETCH_SIZE", fetch)
        _write_counters(run / f"{name}_WRITE_SIZE", write)
    out = bench.record_traffic(run)
    assert out["_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert out["_calibration"]["write_factor"] == pytest.approx(1.0)
    for name, prefixes in bench.TRAFFIC_KERNELS.items():
        n = len(prefixes)   # the decode's call is two kernels, each counted once per call
        assert out[name]["bytes_read"] == pytest.approx(n * 2000.0 * 1024 * 2)
        assert out[name]["bytes_written"] == pytest.approx(n * 4.0 * 1024)
        assert out[name]["source_digest"] == bench.kernel_sources_digest(bench.kernel_sources(W.WORKLOADS[name]))
    assert set(bench.HEADLINE) <= set(bench.TRAFFIC_KERNELS)


def test_more_than_one_gpu_is_refused(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in json.loads(capsys.readouterr().out)["error"]


def test_counter_records_follow_the_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", tmp_path)
    rec = {"source_digest": "abc", "clock_GHz": 2.0, "mfma_busy_frac": 0.5, "executed_over_algorithmic": 1.1,
           "bytes_per_launch": 7.0}
    (tmp_path / "mfma.json").write_text(json.dumps({"w": rec}))
    (tmp_path / "traffic.json").write_text(json.dumps({"w": rec}))
    assert bench.mfma_from_profiles("w", "abc") == {"clock_GHz": 2.0, "mfma_busy_frac": 0.5,
                                                     "executed_over_algorithmic": 1.1}
    assert bench.traffic_from_profiles("w", "abc") == 7.0
    # a changed kernel source, or an unknown workload: no figure
    assert bench.mfma_from_profiles("w", "abd") is None
    assert bench.traffic_from_profiles("w", "abd") is None
    assert bench.mfma_from_profiles("x", "abc") is None


def test_kernel_entry_bounds(monkeypatch):
    # no profiles: the counter fields come back empty
    monkeypatch.setattr(bench, "traffic_from_profiles", lambda *a: None)
    monkeypatch.setattr(bench, "mfma_from_profiles", lambda *a: None)
    # causal GQA prefill: 137.47 GFLOP over 83.9 MB -> the MFMA floor (55 us) is the larger one
    w = W.WORKLOADS["causal_gqa_s4096"]
    fl = 4 * 128 * 32 * 4096 * 4097 / 2
    e = bench.kernel_entry(w, {"seq_lens": None}, 0.110, [0.113, 0.112])
    assert e["bound"] == "mfma" and e["unit"] == "TFLOP/s"
    assert e["achieved"] == pytest.approx(fl / 110e-6 / 1e12)
    assert e["frac"] == pytest.approx(fl / 2.5e15 / 110e-6)
    # banded prefill: 64 FLOP per byte, below the ridge -> the HBM floor
    w = W.WORKLOADS["banded_w128_s8192"]
    by = 4 * 8 * 12 * 8192 * 64 * 2
    e = bench.kernel_entry(w, {"seq_lens": None}, 0.1, [0.1])
    assert e["bound"] == "hbm" and e["unit"] == "GB/s"
    assert e["achieved"] == pytest.approx(by / 100e-6 / 1e9)
    assert e["frac"] == pytest.approx(by / 8e12 / 100e-6)
    # GQA decode: the two caches, 2 GiB, plus Q and O
    w = W.WORKLOADS["gqa_decode_kv8192"]
    e = bench.kernel_entry(w, {}, 0.3, [0.3])
    assert e["bound"] == "hbm"
    assert e["algorithmic_bytes"] == 2 * 64 * 8 * 8192 * 128 * 2 + 2 * 64 * 32 * 128 * 2
    # tiny fp32 prefill: both floors far below a microsecond
    w = W.WORKLOADS["tiny_causal_f32"]
    e = bench.kernel_entry(w, {"seq_lens": None}, 0.005, [0.008, 0.007])
    assert e["bound"] == "latency" and e["kernel_us"] == pytest.approx(5.0)
    assert e["kernel_us_median_single"] == pytest.approx(7.5) and e["kernel_us_min_single"] == pytest.approx(7.0)


def test_headline_is_the_five_configs():
    assert len(bench.HEADLINE) == 5 and all(n in W.WORKLOADS for n in bench.HEADLINE)
    assert bench.HEADLINE_VALUE in bench.HEADLINE and bench.HEADLINE_DECODE in bench.HEADLINE
