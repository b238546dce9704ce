"""GPU parity of the head-dim-32/64 prefill's persistent grid against the fp64 oracle.

That kernel runs as many workgroups as the device holds and deals each a list of q-tiles
(plan::persist_pos): head by head without per-item lengths, and in the order ranked by
each item's costliest q-tile with per-item lengths for at most 64 items (plan::ranked_tile);
past 64 items the lengths are read per q-tile in the head-by-head order.  Every case
here fills the output with NaN before the call, so a q-tile that no list held, or a row
of one that was not written, shows as a non-finite output; every row is then compared
with the oracle (bf16 / fp16: |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise).  Lengths
include empty items, items longer than the keys, and (with a position offset) items whose
rows see no key at all, which the kernel writes as zero q-tiles.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import check, record, to_f64, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mi():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import head_attention_02_amd as m
    m.library()
    return m


@pytest.fixture(scope="module")
def ref():
    return oracle.default()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _lens(seed, n, lo, hi, extra=()):
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi, size=n, endpoint=True)
    for i, v in extra:
        x[i] = v
    return x.astype(np.int32)


def _nan_out(shape, dtype):
    import torch
    t = torch.bfloat16 if dtype == "bf16" else torch.float16
    return torch.full(shape, float("nan"), dtype=t, device="cuda")


PADDED_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, causal, P, (lens seed, lo, hi, fixed entries), W, dtype
    # 64 items: the ranked order, with an empty item and one longer than the keys
    (64, 2, 1, 300, 300, 64, False, 0, (1, 1, 300, ((3, 0), (10, 999))), 0, "bf16"),
    # 65 items: past the ranked order's item count, lengths read per q-tile
    (65, 2, 2, 200, 200, 64, False, 0, (2, 0, 200, ()), 0, "bf16"),
    # causal with a position offset: items with length <= 40 have no row that sees a key
    (40, 4, 2, 260, 300, 32, True, 40, (3, 0, 300, ((0, 40), (1, 41), (2, 12))), 0, "bf16"),
    # a band with lengths, fp16
    (33, 2, 2, 400, 400, 64, False, 0, (4, 1, 400, ()), 96, "f16"),
    # a causal window, GQA 4:1, head dim 32
    (20, 8, 2, 330, 330, 32, True, 0, (5, 1, 330, ()), 70, "bf16"),
]


@pytest.mark.parametrize("case", PADDED_CASES, ids=lambda c: f"B{c[0]}-{c[1]}x{c[2]}-L{c[3]}-D{c[5]}-c{int(c[6])}-P{c[7]}-W{c[9]}-{c[10]}")
def test_persistent_grid_padded(mi, ref, case):
    import torch
    B, Hq, Hkv, Lq, Lk, D, causal, P, (seed, lo, hi, fixed), Wn, dt = case
    say(f"persistent grid, padded: {case}")
    x = W.random_prefill(60 + seed, B, Hq, Hkv, Lq, Lk, D, dt)
    lens = _lens(seed, B, lo, hi, fixed)
    scale = 1.0 / math.sqrt(D)
    out = _nan_out((B, Hq, Lq, D), dt)
    mi.attn_prefill(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), out, pos_offset=P, seq_lens=to_gpu(lens),
                    window=Wn, causal=causal, scale=scale)
    torch.cuda.synchronize()
    g = to_f64(out)
    assert np.all(np.isfinite(g)), "a q-tile of the output was not written"
    want = ref.prefill(x["q"], x["k"], x["v"], scale=scale, causal=causal, pos_offset=P, seq_lens=lens, window=Wn)
    for b in range(B):
        seen_from = max(0, min(int(lens[b]), Lk) - P)
        assert np.all(g[b, :, seen_from:] == 0.0), f"item {b}: rows that see no key must be zero"
    record(f"persistent padded {case[:8]}", check(g, want, dt, f"persistent padded {case}"))


VARLEN_CASES = [
    # item count, Hq, Hkv, D, causal, window, dtype, lens seed, lo, hi
    (64, 4, 2, 64, False, 0, "bf16", 7, 0, 260),
    (70, 2, 2, 64, True, 0, "bf16", 8, 0, 200),
    (48, 4, 4, 32, False, 64, "f16", 9, 1, 300),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"n{c[0]}-{c[1]}x{c[2]}-D{c[3]}-c{int(c[4])}-W{c[5]}-{c[6]}")
def test_persistent_grid_varlen(mi, ref, case):
    import torch
    n, Hq, Hkv, D, causal, Wn, dt, seed, lo, hi = case
    say(f"persistent grid, varlen: {case}")
    lens = _lens(seed, n, lo, hi)
    rng = np.random.default_rng(70 + seed)
    T = int(lens.sum())
    q = W.draw(rng, (T, Hq, D), 1.0, dt)
    k = W.draw(rng, (T, Hkv, D), 1.0, dt)
    v = W.draw(rng, (T, Hkv, D), 1.0, dt)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    scale = 1.0 / math.sqrt(D)
    out = _nan_out((T, Hq, D), dt)
    mi.attn_prefill_varlen(to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(cu), int(lens.max()), out, window=Wn,
                           causal=causal, scale=scale)
    torch.cuda.synchronize()
    g = to_f64(out)
    assert np.all(np.isfinite(g)), "a q-tile of the output was not written"
    want = ref.prefill_varlen(q, k, v, cu, scale=scale, causal=causal, window=Wn)
    record(f"persistent varlen {case[:6]}", check(g, want, dt, f"persistent varlen {case}"))
