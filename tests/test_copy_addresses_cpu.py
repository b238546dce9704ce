"""Host-side bounds check of the kernels' global addresses (no GPU).

`copy_addr_check.cpp` is built with g++ against the kernels' own planning header
(head_attention_02_amd/csrc/tile_plan.hpp) and enumerates, for every launch below, every
block of the grid, every key tile a workgroup visits, every tile-copy instruction and
every lane: the byte offset it computes (whole tiles: per-copy base + per-lane offset;
tail tiles: rows clamped from the tile base) must stay inside the item's valid rows and
the tensor, and the LDS destination inside the tile buffers.  Decode: every cache row a
lane reads stays inside its split's key range.  The launches are every named workload
at full size and every GPU parity shape.  A planted variant (tail rows clamped from each
copy's first row, the addressing that once faulted on a padded batch) must be caught.
"""
import subprocess
from pathlib import Path

import numpy as np
import pytest

import workloads as W

ROOT = Path(__file__).resolve().parent.parent
SRC = Path(__file__).resolve().parent / "copy_addr_check.cpp"
CSRC = ROOT / "head_attention_02_amd" / "csrc"

LAYOUT = {"prefill": 0, "prefill_token_major": 1, "prefill_varlen": 2}
MODE = {"decode": 0, "decode_per_cache": 1, "decode_append": 2}


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = tmp_path_factory.mktemp("addr") / "copy_addr_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", f"-I{CSRC}", str(SRC), "-o", str(exe)], check=True)
    return exe


def run(exe, lines, plant=False):
    args = [str(exe)] + (["--plant"] if plant else [])
    return subprocess.run(args, input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=600)


def prefill_line(layout, B, Hq, Hkv, Lq, Lk, D, P, causal, Wn, lens):
    lens = [] if lens is None else [int(x) for x in lens]
    return " ".join(map(str, ["prefill", layout, B, Hq, Hkv, Lq, Lk, D, P, int(bool(causal)), Wn, len(lens), *lens]))


def decode_line(mode, B, Hq, Hkv, cap, kv_len, D, P, Wn, lens):
    lens = [] if lens is None else [int(x) for x in lens]
    return " ".join(map(str, ["decode", mode, B, Hq, Hkv, cap, kv_len, D, P, Wn, len(lens), *lens]))


def named_lines():
    out = []
    for w in W.WORKLOADS.values():
        lens = W.item_lengths(w)
        if w.dtype == "f32":
            continue   # the fp32 kernel reads K/V rows through bounds-checked plain loads
        if w.kind in LAYOUT:
            Lq, Lk = (int(np.max(lens)),) * 2 if w.kind == "prefill_varlen" else (w.q_len, w.kv_len)
            out.append(prefill_line(LAYOUT[w.kind], w.batch, w.q_heads, w.kv_heads, Lq, Lk, w.head_dim,
                                    w.pos_offset, w.causal, w.window, lens))
        elif w.kind == "decode":
            out.append(decode_line(0, w.batch, w.q_heads, w.kv_heads, w.capacity or w.kv_len, w.kv_len, w.head_dim,
                                   w.pos_offset, w.window, None))
        elif w.kind == "decode_append":
            cl = [w.pos_offset] * w.batch
            out.append(decode_line(2, w.batch, w.q_heads, w.kv_heads, w.capacity or w.kv_len, w.kv_len, w.head_dim,
                                   w.pos_offset, w.window, cl))
    return out


def parity_lines():
    import test_decode_cache_gpu as dc
    import test_layouts_sizes_gpu as ls
    import test_parity_gpu as tp
    import test_varlen_gpu as tv
    out = []
    for B, Hq, Hkv, Lq, Lk, D, causal, P, sl, Wn, dt in tp.PREFILL_CASES:
        out.append(prefill_line(0, B, Hq, Hkv, Lq, Lk, D, P, causal, Wn, sl))
    for B, Hq, Hkv, Lq, Lk, D, causal, P, sl, Wn, dt in ls.TM_CASES:
        out.append(prefill_line(1, B, Hq, Hkv, Lq, Lk, D, P, causal, Wn, sl))
    for lens, Hq, Hkv, D, causal, Wn, dt in tv.VARLEN_CASES:
        out.append(prefill_line(2, len(lens), Hq, Hkv, max(lens), max(lens), D, 0, causal, Wn, lens))
    for B, Hq, Hkv, cap, L, D, P, kl, Wn, dt in tp.DECODE_CASES:
        out.append(decode_line(0, B, Hq, Hkv, cap, L, D, P, Wn, kl))
    for B, Hq, Hkv, cap, D, lens, Wn, dt in dc.PER_ITEM_CASES:
        out.append(decode_line(1, B, Hq, Hkv, cap, cap, D, 0, Wn, lens))
    for B, Hq, Hkv, cap, D, lens, Wn, dt in dc.APPEND_CASES:
        out.append(decode_line(2, B, Hq, Hkv, cap, cap, D, 0, Wn, lens))
    # the size tests: a long cache, a long sequence, 65536 workgroups
    out.append(decode_line(0, 1, 8, 1, 262144, 262144, 128, 0, 0, [262144 - 5]))
    out.append(prefill_line(0, 1, 4, 2, 32768, 32768, 64, 0, True, 0, None))
    lens = W.item_lengths(W.Workload("many", "prefill", 16384, 4, 1, 64, 64, 64, "bf16", 1.0, False,
                                     seq_len_range=(1, 64), seed=53))
    out.append(prefill_line(0, 16384, 4, 1, 64, 64, 64, 0, False, 0, lens))
    # every tail position of a 64-key tile, at every head dim, causal and banded
    for D in (32, 64, 128):
        for Lk in range(193, 257):
            out.append(prefill_line(0, 1, 2, 1, Lk, Lk, D, 0, True, 0, None))
            out.append(prefill_line(1, 2, 2, 2, Lk, Lk, D, 0, False, 50, [Lk, Lk - 100]))
    return out


def test_named_workload_addresses_in_bounds(checker):
    r = run(checker, named_lines())
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


def test_parity_shape_addresses_in_bounds(checker):
    r = run(checker, parity_lines())
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


@pytest.mark.parametrize("D", [32, 64, 128])
def test_planted_block_base_tail_is_caught(checker, D):
    """Tail rows clamped from each copy's first row instead of the tile base: on a
    padded batch whose valid length ends early in a tile, some copy's first row lies past
    the last valid key and its offset goes negative -- the check must report it."""
    lines = [prefill_line(0, 3, 2, 2, 200, 200, D, 0, False, 0, [200, 65, 3])]
    assert run(checker, lines).returncode == 0
    r = run(checker, lines, plant=True)
    assert r.returncode == 1 and "FAIL" in r.stdout, r.stdout


def test_planted_bert_workload_is_caught(checker):
    w = W.WORKLOADS["bert_base_padded"]
    line = prefill_line(0, w.batch, w.q_heads, w.kv_heads, w.q_len, w.kv_len, w.head_dim, 0, False, 0,
                        W.item_lengths(w))
    r = run(checker, [line], plant=True)
    assert r.returncode == 1 and "FAIL" in r.stdout, r.stdout
