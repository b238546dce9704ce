#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass over the whole path on resident synthetic inputs: the five named
configurations, each launched once --
  tiny_causal_f32     causal MHA, fp32, 2 heads, seq 64, head_dim 32 (latency);
  bert_base_padded    encoder, bf16, batch 32, 12 heads, head_dim 64, lengths U{16..512};
  banded_w128_s8192   banded encoder, bf16, batch 8, 12 heads, head_dim 64, |i-j| <= 64;
  causal_gqa_s4096    causal GQA prefill, bf16, 32 query / 8 KV heads, head_dim 128, 4096;
  gqa_decode_kv8192   GQA decode, bf16, batch 64, 32/8 heads, head_dim 128, 8192 keys.
Each configuration in turn runs W warm-up launches and then its K timed launches back to
back, with HIP events recorded on the stream its kernels run on.  Prints one JSON line: `value`
is the causal GQA prefill's throughput in TFLOP/s of algorithmic work (4 * head_dim per
unmasked query-key pair) with its roofline object, the GQA decode's KV-cache bandwidth
rides beside it, and `configs`
holds every configuration's time, rate, roofline fraction (against the larger of its MFMA
and HBM floors) and oracle baseline.  `--workload` benchmarks one named workload alone.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

`--workload copy_calibration` runs a plain 1 GiB device copy instead, the known-size
reference against which the rocprofv3 FETCH_SIZE / WRITE_SIZE counters are scaled;
`--record-traffic DIR` (no GPU) turns those counter runs into profiles/traffic.json, and
`--record-mfma DIR` (no GPU) turns one matrix-core counter run per prefill workload into
profiles/mfma.json (clock, MFMA busy share, executed against algorithmic FLOPs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 (and fp16) MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (vector)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PROFILES = ROOT / "profiles"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work


def keys_per_row(w: W.Workload, seq_lens) -> np.ndarray:
    """Number of keys in the key set of every query row: [batch, q_len]."""
    pos = w.pos_offset + np.arange(w.q_len)
    counts = np.zeros((w.batch, w.q_len), np.int64)
    for b in range(w.batch):
        valid = w.kv_len if seq_lens is None else min(max(int(seq_lens[b]), 0), w.kv_len)
        if w.causal:
            hi = np.minimum(pos, valid - 1)
            lo = np.zeros_like(pos) if w.window == 0 else np.maximum(0, pos - w.window + 1)
        else:
            hi = np.full_like(pos, valid - 1) if w.window == 0 else np.minimum(valid - 1, pos + w.window // 2)
            lo = np.zeros_like(pos) if w.window == 0 else np.maximum(0, pos - w.window // 2)
        c = np.maximum(0, hi - lo + 1)
        c[pos >= valid] = 0
        counts[b] = c
    return counts


def prefill_flops(w: W.Workload, seq_lens) -> float:
    return 4.0 * w.head_dim * w.q_heads * float(keys_per_row(w, seq_lens).sum())


def prefill_bytes(w: W.Workload, seq_lens) -> float:
    """Q + valid K/V rows + O, each once."""
    esz = 4 if w.dtype == "f32" else 2
    if w.kind == "prefill_varlen":   # every token row is an item's
        return 2.0 * (w.q_heads + w.kv_heads) * w.head_dim * esz * float(np.sum(seq_lens))
    valid = np.full(w.batch, w.kv_len) if seq_lens is None else np.clip(seq_lens, 0, w.kv_len)
    kv = 2.0 * w.kv_heads * w.head_dim * esz * float(valid.sum())
    qo = 2.0 * w.batch * w.q_heads * w.q_len * w.head_dim * esz
    return kv + qo


def decode_bytes(w: W.Workload) -> float:
    esz = 4 if w.dtype == "f32" else 2
    keys = min(w.pos_offset + 1, w.kv_len)
    kv = 2.0 * w.batch * w.kv_heads * keys * w.head_dim * esz
    qo = 2.0 * w.batch * w.q_heads * w.head_dim * esz
    return kv + qo


def decode_flops(w: W.Workload) -> float:
    return 4.0 * w.head_dim * w.batch * w.q_heads * min(w.pos_offset + 1, w.kv_len)


# ---------------------------------------------------------------------------
# device side


def to_gpu(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


class Runner:
    """Holds one workload's resident device inputs and launches it."""

    def __init__(self, w: W.Workload, x: dict):
        import torch
        import head_attention_02_amd as mi
        self.mi, self.w = mi, w
        self.q, self.k, self.v = to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"])
        self.out = torch.empty_like(self.q)
        lens = x.get("seq_lens") if w.kind in ("prefill", "prefill_token_major") else x.get("kv_lens")
        if w.kind == "prefill_varlen":
            self.cu = to_gpu(x["cu_seqlens"])
            self.max_seqlen = int(np.max(x["seq_lens"]))
        self.lens = None if lens is None else to_gpu(lens)
        self.ws = None
        if w.kind in ("decode", "decode_append"):
            n = mi.attn_decode_workspace_bytes(w.batch, w.q_heads, w.kv_heads, w.kv_len, w.head_dim)
            self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
        if w.kind == "decode_append":
            self.k_new, self.v_new = to_gpu(x["k_new"]), to_gpu(x["v_new"])
            self.lens = to_gpu(x["cache_lens"])
            self.k_table, self.v_table = mi.CacheTable(self.k), mi.CacheTable(self.v)

    def __call__(self):
        w = self.w
        if w.kind == "prefill":
            self.mi.attn_prefill(self.q, self.k, self.v, self.out, pos_offset=w.pos_offset, seq_lens=self.lens,
                                 window=w.window, causal=w.causal, scale=w.attn_scale)
        elif w.kind == "prefill_token_major":
            self.mi.attn_prefill_token_major(self.q, self.k, self.v, self.out, pos_offset=w.pos_offset,
                                             seq_lens=self.lens, window=w.window, causal=w.causal, scale=w.attn_scale)
        elif w.kind == "prefill_varlen":
            self.mi.attn_prefill_varlen(self.q, self.k, self.v, self.cu, self.max_seqlen, self.out, window=w.window,
                                        causal=w.causal, scale=w.attn_scale)
        elif w.kind == "decode_append":
            # the same slot is rewritten every step (the lengths are not advanced), so
            # every step does the same work
            self.mi.attn_decode_append(self.q, self.k_new, self.v_new, self.k_table, self.v_table, self.lens,
                                       self.out, window=w.window, scale=w.attn_scale, workspace=self.ws)
        else:
            self.mi.attn_decode(self.q, self.k, self.v, self.out, kv_len=w.kv_len, pos_offset=w.pos_offset,
                                kv_lens=self.lens, window=w.window, scale=w.attn_scale, workspace=self.ws)


def kernel_sources_digest(names) -> str:
    h = hashlib.sha256()
    for n in names:
        h.update((ROOT / "head_attention_02_amd" / "csrc" / n).read_bytes())
    return h.hexdigest()[:16]


def traffic_from_profiles(key: str, digest: str):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic.json), or
    None when the kernel source changed since the counters were taken."""
    f = PROFILES / "traffic.json"
    if not f.exists():
        return None
    rec = json.loads(f.read_text()).get(key)
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def mfma_from_profiles(key: str, digest: str):
    """Matrix-core counters of a prefill launch (profiles/mfma.json): clock, busy share and
    executed / algorithmic FLOPs, or None when the kernel source changed since."""
    f = PROFILES / "mfma.json"
    if not f.exists():
        return None
    rec = json.loads(f.read_text()).get(key)
    if not rec or rec.get("source_digest") != digest:
        return None
    return {k: rec[k] for k in ("clock_GHz", "mfma_busy_frac", "executed_over_algorithmic")}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, timed on the host cores on a bounded sample


def cpu_baseline_varlen(w: W.Workload, x: dict, budget_s: float) -> dict:
    """The oracle on the first n items of the unpadded batch (whole items: the oracle
    has no per-row entry for this layout)."""
    import oracle
    ref = oracle.default()
    nt = len(os.sched_getaffinity(0))
    lens, cu = np.asarray(x["seq_lens"], np.int64), np.asarray(x["cu_seqlens"], np.int64)
    n = 1
    while True:
        T = int(cu[n])
        t0 = time.perf_counter()
        ref.prefill_varlen(x["q"][:T], x["k"][:T], x["v"][:T], cu[:n + 1].astype(np.int32), scale=w.attn_scale,
                           causal=w.causal, window=w.window, nthreads=nt)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or n == w.batch:
            break
        n = min(w.batch, max(n * 2, int(n * budget_s / max(dt, 1e-3))))
    sub = W.Workload(w.name, "prefill", n, w.q_heads, w.kv_heads, w.q_len, w.kv_len, w.head_dim, w.dtype, w.sigma,
                     w.causal, window=w.window)
    flops = prefill_flops(sub, lens[:n])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": ref.threads_used, "kind": "oracle",
            "sample": f"the first {n} of {w.batch} items of {w.name} ({T} tokens), fp64, {dt:.1f} s"}


def cpu_baseline_prefill(w: W.Workload, x: dict, budget_s: float) -> dict:
    import oracle
    if w.kind == "prefill_varlen":
        return cpu_baseline_varlen(w, x, budget_s)
    if w.kind == "prefill_token_major":   # the oracle's rows entry reads head-major arrays
        x = dict(x, **{n: np.ascontiguousarray(x[n].transpose(0, 2, 1, 3)) for n in ("q", "k", "v")})
    ref = oracle.default()
    nt = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(123)
    total = w.batch * w.q_heads * w.q_len
    perm = rng.permutation(total)
    rows_all = np.stack([perm // (w.q_heads * w.q_len), (perm // w.q_len) % w.q_heads, perm % w.q_len], 1)
    counts = keys_per_row(w, x["seq_lens"])
    kw = dict(scale=w.attn_scale, causal=w.causal, pos_offset=w.pos_offset, seq_lens=x["seq_lens"], window=w.window)
    n = min(64, total)
    while True:
        rows = rows_all[:n].astype(np.int32)
        t0 = time.perf_counter()
        ref.prefill(x["q"], x["k"], x["v"], rows=rows, nthreads=nt, **kw)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or n == total:
            break
        n = min(total, max(n * 2, int(n * budget_s / max(dt, 1e-3))))
    flops = 4.0 * w.head_dim * float(counts[rows[:, 0], rows[:, 2]].sum())
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": ref.threads_used, "kind": "oracle",
            "sample": f"{n} of {total} query rows of {w.name} (uniform random), fp64, {dt:.1f} s"}


def cpu_baseline_decode(w: W.Workload, x: dict, budget_s: float) -> dict:
    import oracle
    ref = oracle.default()
    nt = len(os.sched_getaffinity(0))
    total = w.batch * w.q_heads
    rng = np.random.default_rng(321)
    perm = rng.permutation(total)
    pairs_all = np.stack([perm // w.q_heads, perm % w.q_heads], 1)
    n = min(8, total)
    while True:
        pairs = pairs_all[:n].astype(np.int32)
        t0 = time.perf_counter()
        if w.kind == "decode_append":
            # the oracle's two steps: copy the caches with the new rows in, then attend
            ref.decode_append(x["q"], x["k_new"], x["v_new"], list(x["k"]), list(x["v"]), x["cache_lens"],
                              scale=w.attn_scale, window=w.window, rows=pairs, nthreads=nt)
        else:
            ref.decode(x["q"], x["k"], x["v"], kv_len=w.kv_len, scale=w.attn_scale, pos_offset=w.pos_offset,
                       window=w.window, rows=pairs, nthreads=nt)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or n == total:
            break
        n = min(total, max(n * 2, int(n * budget_s / max(dt, 1e-3))))
    esz = 4 if w.dtype == "f32" else 2
    # bytes of K and V each query row streams (the GPU reads each once per KV head group)
    by = 2.0 * n * min(w.pos_offset + 1, w.kv_len) * w.head_dim * esz
    return {"value": by / dt / 1e9, "unit": "GB/s", "cores": ref.threads_used, "kind": "oracle",
            "sample": f"{n} of {total} (item, query head) rows of {w.name}, fp64, {dt:.1f} s"}


# ---------------------------------------------------------------------------
# HBM counter calibration: a plain device-to-device copy of a known size


COPY_BYTES = 1 << 30


def copy_calibration(steps: int, warmup: int) -> int:
    """Copies 1 GiB between two device buffers `steps` times.  Under rocprofv3 --pmc the
    FETCH_SIZE / WRITE_SIZE this copy reports, against its known 1 GiB read and 1 GiB
    written, gives the factor that turns those counters into bytes for the attention
    kernels measured the same way."""
    import torch
    src = torch.full((COPY_BYTES,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    begin, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    begin.record()
    for _ in range(steps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = begin.elapsed_time(end) / max(steps, 1)
    print(json.dumps({"workload": "copy_calibration", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                      "ms_per_copy": ms, "GBps": 2 * COPY_BYTES / (ms / 1e3) / 1e9}), flush=True)
    return 0


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counter runs -> profiles/traffic.json

# The workloads whose HBM traffic is recorded (one rocprofv3 --pmc run per counter each,
# under DIR/<workload>_<COUNTER>) and the kernel-name prefixes that make up one call.
TRAFFIC_KERNELS = {
    "tiny_causal_f32": ["prefill_f32_kernel<32"],
    "bert_base_padded": ["prefill_bf16_narrow_kernel<64"],
    "banded_w128_s8192": ["prefill_bf16_narrow_kernel<64"],
    "gqa_decode_kv8192": ["decode_split_kernel<128", "decode_combine_kernel<128"],
    "causal_gqa_s4096": ["prefill_bf16_kernel<128"],
    "gqa_decode_append_kv8192": ["decode_split_kernel<128", "decode_combine_kernel<128"],
}


def _counter_rows(run_dir: Path, counter: str):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc csv run."""
    import csv
    files = sorted(run_dir.rglob("*counter_collection.csv"))
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def _per_dispatch(rows, prefix: str) -> float:
    vals = [v for name, v in rows if prefix in name]
    return float(np.mean(vals)) if vals else 0.0


def record_traffic(run_root: Path) -> dict:
    """Reads <run_root>/<workload>_{FETCH_SIZE,WRITE_SIZE} for every workload of
    TRAFFIC_KERNELS and <run_root>/copy_{FETCH_SIZE,WRITE_SIZE} (one rocprofv3 --pmc run
    each) and writes profiles/traffic.json: HBM bytes per call of each workload, with the
    counters scaled by what they read for the 1 GiB copy."""
    cf = _per_dispatch(_counter_rows(run_root / "copy_FETCH_SIZE", "FETCH_SIZE"), "copyBuffer")
    cw = _per_dispatch(_counter_rows(run_root / "copy_WRITE_SIZE", "WRITE_SIZE"), "copyBuffer")
    ff, wf = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    out = {"_calibration": {"kernel": "__amd_rocclr_copyBuffer", "bytes_read": COPY_BYTES,
                            "bytes_written": COPY_BYTES, "FETCH_SIZE_KiB": cf, "WRITE_SIZE_KiB": cw,
                            "fetch_factor": ff, "write_factor": wf}}
    for name, prefixes in TRAFFIC_KERNELS.items():
        fr = _counter_rows(run_root / f"{name}_FETCH_SIZE", "FETCH_SIZE")
        wr = _counter_rows(run_root / f"{name}_WRITE_SIZE", "WRITE_SIZE")
        fk = sum(_per_dispatch(fr, p) for p in prefixes)
        wk = sum(_per_dispatch(wr, p) for p in prefixes)
        rd, wt = fk * 1024 * ff, wk * 1024 * wf
        out[name] = {"source_digest": kernel_sources_digest(kernel_sources(W.WORKLOADS[name])), "kernels": prefixes,
                     "FETCH_SIZE_KiB": fk, "WRITE_SIZE_KiB": wk, "bytes_read": rd, "bytes_written": wt,
                     "bytes_per_launch": rd + wt}
    (PROFILES / "traffic.json").write_text(json.dumps(out, indent=1) + "\n")
    return out


# ---------------------------------------------------------------------------
# Matrix-core use from rocprofv3 counter runs -> profiles/mfma.json

# (workload, kernel-name prefix); one --pmc run each, under DIR/<workload>
MFMA_RUNS = [
    ("causal_gqa_s4096", "prefill_bf16_kernel<128"),
    ("causal_gqa_s4096_f16", "prefill_bf16_kernel<128"),
    ("banded_w128_s8192", "prefill_bf16_narrow_kernel<64"),
    ("bert_base_padded", "prefill_bf16_narrow_kernel<64"),
    ("bert_base_varlen", "prefill_bf16_narrow_kernel<64"),
]
MFMA_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU"]
XCDS, SIMDS = 8, 256 * 4            # MI355X: 8 XCDs, 256 CUs of 4 SIMDs
MFMA_FLOP_PER_SIMD_CYCLE = 1024     # 16-bit dense: 32x32x16 MFMA (32768 FLOP) per 32 cycles


def _per_dispatch_with_time(run_dir: Path, prefix: str) -> dict:
    """Mean counter values and mean duration (us) over the dispatches whose name has prefix."""
    import csv
    files = sorted(run_dir.rglob("*counter_collection.csv"))
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    vals: dict = {}
    durs: dict = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if prefix not in r["Kernel_Name"]:
                    continue
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                durs[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    if not durs:
        raise ValueError(f"no dispatch of {prefix} under {run_dir}")
    out = {k: float(np.mean(v)) for k, v in vals.items()}
    out["duration_us"] = float(np.mean(list(durs.values())))
    out["dispatches"] = len(durs)
    return out


def record_mfma(run_root: Path) -> dict:
    """Reads one rocprofv3 --pmc run of MFMA_COUNTERS per workload of MFMA_RUNS (directory
    <run_root>/<workload>) and writes profiles/mfma.json: per launch, the shader clock
    (GRBM_GUI_ACTIVE counts the cycles of all 8 XCDs), the share of each SIMD's cycles its
    matrix core was busy (SQ_VALU_MFMA_BUSY_CYCLES sums the 1024 SIMDs), VALU instructions
    per SIMD, the MFMA FLOPs executed (busy cycles x 1024 FLOP) against the algorithmic
    FLOPs, and the algorithmic rate against the 16-bit dense peak."""
    out = {"_counters": MFMA_COUNTERS, "_simds": SIMDS, "_xcds": XCDS,
           "_flop_per_busy_cycle": MFMA_FLOP_PER_SIMD_CYCLE, "_peak_TFLOPs": PEAK_BF16_TFLOPS}
    for name, prefix in MFMA_RUNS:
        w = W.WORKLOADS[name]
        src = kernel_sources(w)
        seq_lens = W.make_inputs(w)["seq_lens"] if w.seq_len_range is not None else None
        c = _per_dispatch_with_time(run_root / name, prefix)
        us = c["duration_us"]
        cyc = c["GRBM_GUI_ACTIVE"] / XCDS
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS
        executed = busy * SIMDS * MFMA_FLOP_PER_SIMD_CYCLE
        alg = prefill_flops(w, seq_lens)
        out[name] = {"source_digest": kernel_sources_digest(src), "kernel": prefix,
                     "dispatches": c["dispatches"], "duration_us": us, "clock_GHz": cyc / (us * 1e3),
                     "cycles": cyc, "mfma_busy_cycles_per_simd": busy, "mfma_busy_frac": busy / cyc,
                     "valu_insts_per_simd": c["SQ_ACTIVE_INST_VALU"] / SIMDS,
                     "executed_mfma_flop": executed, "algorithmic_flop": alg,
                     "executed_over_algorithmic": executed / alg,
                     "algorithmic_TFLOPs": alg / (us * 1e-6) / 1e12,
                     "frac_of_peak": alg / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}
    (PROFILES / "mfma.json").write_text(json.dumps(out, indent=1) + "\n")
    return out


# ---------------------------------------------------------------------------


# The five named configurations of one step; `value` is the causal GQA prefill's, the
# decode fields the GQA decode's.  The two headline workloads are timed first.
HEADLINE = ("causal_gqa_s4096", "gqa_decode_kv8192", "tiny_causal_f32", "bert_base_padded", "banded_w128_s8192")
HEADLINE_VALUE = "causal_gqa_s4096"
HEADLINE_DECODE = "gqa_decode_kv8192"


def kernel_sources(w: W.Workload):
    if w.kind in ("decode", "decode_append"):
        return ["decode.hip", "mi_attn_device.hpp", "mi_attn_kernels.hpp"]
    if w.dtype == "f32":
        return ["prefill_f32.hip", "mi_attn_device.hpp", "mi_attn_kernels.hpp"]
    if w.head_dim == 128:
        return ["prefill_bf16.hip", "mi_attn_device.hpp", "mi_attn_kernels.hpp"]
    return ["prefill_bf16_narrow.hip", "mi_attn_device.hpp", "mi_attn_kernels.hpp"]


def kernel_entry(w: W.Workload, x: dict, mean_ms: float, times_ms) -> dict:
    """One workload's figures: mean_ms, the mean launch time of K launches back to back (one
    event pair around them), gives the rate of algorithmic work and the roofline fraction
    -- the larger of the two floors (FLOPs at the MFMA peak, bytes at the HBM peak) over
    the measured time; `bound` names the floor that is larger.  times_ms, the launches of a
    second pass timed one by one (an event between every two, which adds a few
    microseconds to each), give the median and the minimum.  A workload below a
    microsecond of floor is latency-bound: its fraction is given, but the time is what
    counts."""
    ms = float(mean_ms)
    sec = ms / 1e3
    src = kernel_sources(w)
    if w.kind in ("decode", "decode_append"):
        fl, by = decode_flops(w), decode_bytes(w)
    else:
        fl, by = prefill_flops(w, x["seq_lens"]), prefill_bytes(w, x["seq_lens"])
    peak_f = PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS   # fp16 dense = bf16 dense
    t_mfma, t_hbm = fl / (peak_f * 1e12), by / (PEAK_HBM_GBPS * 1e9)
    floor = max(t_mfma, t_hbm)
    if floor < 1e-6:
        bound = "latency"
    else:
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
    if bound == "hbm":
        achieved, peak, unit = by / sec / 1e9, PEAK_HBM_GBPS, "GB/s"
    else:
        achieved, peak, unit = fl / sec / 1e12, peak_f, "TFLOP/s"
    e = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": floor / sec,
         "traffic": traffic_from_profiles(w.name, kernel_sources_digest(src)),
         "kernel_us": ms * 1e3, "kernel_us_median_single": float(np.median(times_ms)) * 1e3,
         "kernel_us_min_single": float(np.min(times_ms)) * 1e3,
         "TFLOPs": fl / sec / 1e12, "frac_of_mfma_peak": fl / sec / 1e12 / peak_f,
         "GBps": by / sec / 1e9, "frac_of_hbm_peak": by / sec / 1e9 / PEAK_HBM_GBPS,
         "algorithmic_flop": fl, "algorithmic_bytes": by,
         "floor_us": {"mfma": t_mfma * 1e6, "hbm": t_hbm * 1e6}}
    if w.kind not in ("decode", "decode_append"):
        e["mfma_counters"] = mfma_from_profiles(w.name, kernel_sources_digest(src))
    return e


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="headline",
                    help="headline (the five configurations of one step), a name in "
                         "workloads.WORKLOADS, or copy_calibration (1 GiB device copy for the HBM counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the causal GQA prefill and GQA decode baselines "
                         "(half that for the other three)")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="no GPU run: turn the rocprofv3 FETCH_SIZE / WRITE_SIZE runs under DIR into "
                         "profiles/traffic.json")
    ap.add_argument("--record-mfma", metavar="DIR",
                    help="no GPU run: turn the rocprofv3 matrix-core counter runs under DIR into "
                         "profiles/mfma.json")
    args = ap.parse_args()
    if args.record_mfma:
        print(json.dumps(record_mfma(Path(args.record_mfma)), indent=1))
        return 0
    if args.record_traffic:
        print(json.dumps(record_traffic(Path(args.record_traffic)), indent=1))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this attention library runs on one GPU; --gpus must be 1"}))
        return 2

    import torch
    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    import head_attention_02_amd as mi
    mi.library()

    if args.workload == "copy_calibration":
        return copy_calibration(args.steps, args.warmup)
    if args.workload == "headline":
        names = list(HEADLINE)
    else:
        names = [args.workload]
    ws = [W.WORKLOADS[n] for n in names]
    inputs, runners = [], []
    for w in ws:
        log(f"generating {w.name}")
        x = W.make_inputs(w)
        inputs.append(x)
        runners.append(Runner(w, x))
    torch.cuda.synchronize()

    # Each workload in turn: W warm-up launches, then K timed launches back to back with one
    # event before and one after them, so that a workload is timed in the clock and cache
    # state its own launches leave (the chip's clock follows the power of the last
    # milliseconds of work: a causal prefill launched right after milliseconds of HBM-bound
    # decode ran its first launches 20 % slower).  The K launches of all workloads are the K
    # steps of the timed region.  A second pass, after the timed region, times K launches of
    # each workload one by one for the spread (an event between every two launches adds a
    # few microseconds to each, so the mean comes from the first pass).
    K = args.steps
    spans = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in runners]
    begin, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    begin.record()
    for i, r in enumerate(runners):
        for _ in range(args.warmup):
            r()
        torch.cuda._sleep(1_000_000)   # keep the queue ahead of the GPU so events time kernels, not launches
        spans[i][0].record()
        for s in range(K):
            r()
        spans[i][1].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_ms = [a.elapsed_time(b) / K for a, b in spans]
    step_ms = sum(mean_ms)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(K + 1)] for _ in runners]
    for i, r in enumerate(runners):
        for _ in range(args.warmup):
            r()
        torch.cuda._sleep(1_000_000)
        ev[i][0].record()
        for s in range(K):
            r()
            ev[i][s + 1].record()
    torch.cuda.synchronize()
    per_launch = [[ev[i][s].elapsed_time(ev[i][s + 1]) for s in range(K)] for i in range(len(runners))]

    result = {"metric": "attention TFLOP/s (prefill, % MFMA peak); decode KV GB/s (% HBM peak)",
              "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": step_ms,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "data": "synthetic (seeded N(0, sigma^2), bf16 by round-to-nearest-even)"}
    rooflines = {w.name: kernel_entry(w, x, m, t) for w, x, m, t in zip(ws, inputs, mean_ms, per_launch)}
    head = ws[0] if args.workload != "headline" else W.WORKLOADS[HEADLINE_VALUE]
    r0 = rooflines[head.name]
    result["value"] = r0["achieved"]
    result["unit"] = r0["unit"]
    result["dtype"] = head.dtype
    result["roofline"] = {k: r0[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    if args.workload == "headline":
        r1 = rooflines[HEADLINE_DECODE]
        result["decode_kv_GBps"] = r1["achieved"]
        result["roofline_decode"] = {k: r1[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    result["config"] = {"workload": " + ".join(f"{w.kind} {w.name}" for w in ws),
                        "value_from": head.name,
                        "detail": {w.name: {"batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                                            "q_len": w.q_len, "kv_len": w.kv_len, "head_dim": w.head_dim,
                                            "causal": w.causal, "window": w.window, "pos_offset": w.pos_offset,
                                            "dtype": w.dtype} for w in ws}}
    result["configs"] = rooflines
    result["wall_s_timed_region"] = wall

    if not args.no_cpu_baseline:
        log("timing the oracle on the host (cpu_baseline)")
        for w, x in zip(ws, inputs):
            budget = args.cpu_budget if w.name in (head.name, HEADLINE_DECODE) else args.cpu_budget / 2
            if w.kind in ("prefill", "prefill_token_major", "prefill_varlen"):
                cb = cpu_baseline_prefill(w, x, budget)
            else:
                cb = cpu_baseline_decode(w, x, budget)
            rooflines[w.name]["cpu_baseline"] = cb
        result["cpu_baseline"] = rooflines[head.name]["cpu_baseline"]
        if HEADLINE_DECODE in rooflines and head.name != HEADLINE_DECODE:
            result["cpu_baseline_decode"] = rooflines[HEADLINE_DECODE]["cpu_baseline"]
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
