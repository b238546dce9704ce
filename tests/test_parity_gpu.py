"""GPU parity: libmi_attn (through its C ABI) against the fp64 oracle, element by element.

Sizes span several tiles with ragged tails; the five named workloads run at full size
in the launch configuration the benchmark times, and every output element of them is
compared with the oracle.  bf16: |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise; fp32:
max abs 1e-4.  The named workloads' error margins are recorded (gpu_util.record).
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


def poison(arrays, lens, axis_len_dim, dtype):
    """Write NaN into every position at or past each item's length (dim 2)."""
    nan = W.BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    for a in arrays:
        for b, n in enumerate(lens):
            a[b, :, max(int(n), 0):] = nan


# ---------------------------------------------------------------------------
# prefill: assorted shapes

PREFILL_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, causal, P, seq_lens, W, dtype
    (2, 4, 4, 300, 300, 64, False, 0, None, 0, "bf16"),
    (1, 8, 2, 257, 257, 128, True, 0, None, 0, "bf16"),
    (2, 4, 1, 129, 400, 128, True, 271, None, 0, "bf16"),
    (3, 6, 3, 200, 200, 32, False, 0, [200, 1, 0], 0, "bf16"),
    (2, 4, 4, 333, 333, 64, False, 0, None, 128, "bf16"),
    (1, 4, 4, 300, 300, 64, False, 0, None, 7, "bf16"),
    (1, 8, 1, 190, 190, 128, True, 0, None, 50, "bf16"),
    (2, 2, 2, 100, 150, 64, True, 50, [150, 120], 0, "bf16"),
    (4, 4, 2, 64, 64, 128, False, 0, [64, 37, 1, 999], 0, "bf16"),
    (1, 2, 2, 1, 1, 64, True, 0, None, 0, "bf16"),
    (1, 16, 2, 130, 130, 32, True, 0, [97], 33, "bf16"),
    (2, 4, 2, 150, 150, 64, True, 0, None, 0, "f32"),
    (1, 2, 2, 70, 90, 128, False, 20, [85], 9, "f32"),
    (1, 4, 4, 100, 100, 32, True, 0, None, 16, "f32"),
    (3, 3, 1, 65, 65, 128, False, 0, [65, 0, 13], 0, "f32"),
    # several 256-row q-tiles at head dim 128, bidirectional, banded, and with the
    # (item, kv head) unit count a multiple of 8 (the XCD-grouped block order)
    (1, 8, 2, 520, 700, 128, False, 0, None, 0, "bf16"),
    (1, 4, 2, 600, 600, 128, False, 0, None, 200, "bf16"),
    (2, 8, 4, 300, 300, 128, True, 0, None, 0, "bf16"),
    (2, 8, 4, 300, 300, 64, True, 0, [300, 257], 0, "bf16"),
    # fp16 inputs (the fp16 MFMA and fp16 rounding of P and the output)
    (1, 8, 2, 257, 257, 128, True, 0, None, 0, "f16"),
    (1, 4, 2, 600, 600, 128, False, 0, [555], 200, "f16"),
    (2, 4, 4, 333, 333, 64, False, 0, None, 128, "f16"),
    (3, 6, 3, 200, 200, 32, False, 0, [200, 1, 0], 0, "f16"),
    (2, 2, 2, 100, 150, 64, True, 50, [150, 120], 0, "f16"),
    # head dims 32/64 with narrow bands over long sequences (many q-tiles per workgroup
    # list of the persistent grid): GQA and a padded item; a causal window; a position
    # offset with fp16; a causal window one key wider than the bidirectional one; a band
    # wider than a q-tile
    (2, 6, 2, 9000, 9000, 64, False, 0, [9000, 8100], 128, "bf16"),
    (1, 4, 4, 5000, 5000, 32, True, 0, None, 96, "bf16"),
    (1, 8, 8, 3000, 3100, 64, False, 100, None, 64, "f16"),
    (2, 4, 4, 777, 777, 64, True, 0, [777, 500], 129, "bf16"),
    (1, 2, 2, 700, 700, 64, False, 0, None, 300, "bf16"),
    # one KV head for many query heads (32:1 and 16:1)
    (2, 32, 1, 300, 300, 128, True, 0, None, 0, "bf16"),
    (3, 16, 1, 200, 200, 64, False, 0, [200, 77, 130], 0, "bf16"),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-c{int(c[6])}-P{c[7]}-W{c[9]}-{c[10]}")
def test_prefill_parity(mi, ref, case):
    B, Hq, Hkv, Lq, Lk, D, causal, P, sl, Wn, dt = case
    say(f"prefill case {case}")
    x = W.random_prefill(7, B, Hq, Hkv, Lq, Lk, D, dt)
    q, k, v = x["q"], x["k"], x["v"]
    seq = None if sl is None else np.array(sl, np.int32)
    if seq is not None:
        poison([k, v], np.minimum(seq, Lk), 2, dt)
        poison([q], np.clip(seq - P, 0, Lq), 2, dt)
    scale = 1.0 / math.sqrt(D)
    want = ref.prefill(q, k, v, scale=scale, causal=causal, pos_offset=P, seq_lens=seq, window=Wn)
    got = mi.attn_prefill(to_gpu(q), to_gpu(k), to_gpu(v), pos_offset=P,
                          seq_lens=None if seq is None else to_gpu(seq), window=Wn, causal=causal, scale=scale)
    import torch
    torch.cuda.synchronize()
    g = to_f64(got)
    if seq is not None:
        for b in range(B):
            pad_from = max(0, min(int(seq[b]), Lk) - P)
            assert np.all(g[b, :, pad_from:] == 0.0), "padded query rows must be zero"
    check(g, want, dt, f"prefill {case}")


# ---------------------------------------------------------------------------
# decode: assorted shapes

DECODE_CASES = [
    # B, Hq, Hkv, cap, kv_len, D, P, kv_lens, W, dtype
    (4, 32, 8, 1024, 1000, 128, 999, None, 0, "bf16"),
    (5, 8, 8, 700, 700, 64, 300, None, 0, "bf16"),
    (6, 16, 2, 2048, 2000, 128, 0, [2000, 1, 0, 1500, 1999, 777], 0, "bf16"),
    (3, 12, 4, 512, 512, 32, 0, [512, 100, 3], 64, "bf16"),
    (2, 8, 1, 333, 333, 128, 332, None, 1, "bf16"),
    (2, 4, 1, 300, 300, 128, 299, None, 17, "f32"),
    (2, 6, 2, 256, 200, 64, 0, [200, 50], 0, "f32"),
    # 512 (item, kv head) units: one workgroup per key range, no split and no combine pass
    (64, 8, 8, 96, 90, 64, 0, [(37 * i) % 91 for i in range(64)], 0, "f32"),
    (128, 8, 4, 64, 64, 128, 40, None, 9, "bf16"),
    (4, 32, 8, 1024, 1000, 128, 999, None, 0, "f16"),
    (3, 12, 4, 512, 512, 32, 0, [512, 100, 3], 64, "f16"),
    # one KV head for 32 query heads: four groups of 8 heads per key range
    (2, 32, 1, 600, 600, 128, 0, [600, 301], 0, "bf16"),
    (3, 32, 1, 400, 400, 64, 399, None, 100, "f16"),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-P{c[6]}-W{c[8]}-{c[9]}")
def test_decode_parity(mi, ref, case):
    B, Hq, Hkv, cap, L, D, P, kl, Wn, dt = case
    say(f"decode case {case}")
    x = W.random_decode(11, B, Hq, Hkv, cap, D, dt)
    q, k, v = x["q"], x["k"], x["v"]
    lens = np.array(kl, np.int32) if kl is not None else None
    poison([k, v], lens if lens is not None else [L] * B, 2, dt)
    scale = 1.0 / math.sqrt(D)
    want = ref.decode(q, k, v, kv_len=L, scale=scale, pos_offset=P, kv_lens=lens, window=Wn)
    got = mi.attn_decode(to_gpu(q), to_gpu(k), to_gpu(v), kv_len=L, pos_offset=P,
                         kv_lens=None if lens is None else to_gpu(lens), window=Wn, scale=scale)
    import torch
    torch.cuda.synchronize()
    check(to_f64(got), want, dt, f"decode {case}")


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_prefill_nonpositive_scale(mi, ref, D, scale):
    """scale <= 0 takes the kernels' other softmax form (scale applied before the max);
    scale 0 makes every visible key equally likely."""
    say(f"prefill scale {scale} D {D}")
    x = W.random_prefill(13, 2, 4, 2, 270, 270, D, "bf16")
    want = ref.prefill(x["q"], x["k"], x["v"], scale=scale, causal=True, window=100)
    got = mi.attn_prefill(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), causal=True, window=100, scale=scale)
    import torch
    torch.cuda.synchronize()
    check(to_f64(got), want, "bf16", f"scale {scale} D {D}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("scale", [0.05, 0.5, 1.0 / math.log2(math.e), 0.75, 2.0])
def test_prefill_positive_scales(mi, ref, D, dtype, scale):
    """Positive scales on both sides of scale * log2(e) = 1: below it the fp16 kernels may
    carry the scale in Q, above it they keep it out (c * q could overflow fp16); bf16
    carries it at any positive scale."""
    say(f"prefill scale {scale:.4f} {dtype} D {D}")
    x = W.random_prefill(17, 1, 4, 2, 230, 230, D, dtype, sigma=0.5)
    want = ref.prefill(x["q"], x["k"], x["v"], scale=scale, causal=True)
    got = mi.attn_prefill(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), causal=True, scale=scale)
    import torch
    torch.cuda.synchronize()
    check(to_f64(got), want, dtype, f"scale {scale:.4f} {dtype} D {D}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_running_max_keeps_moving(mi, ref, D, dtype, causal):
    """Scores that grow by about 10 (log2 units) per 64 keys: every row's running max
    moves past the lazy-rescale slack on nearly every key tile, so the rescale path (O and
    the row sum scaled down, the tile's exponents re-referenced to the new max) runs
    tile after tile instead of once."""
    say(f"prefill growing scores {dtype} D {D} causal {causal}")
    rng = np.random.default_rng(23)
    L, scale = 300, 1.0 / math.sqrt(D)
    u = np.full(D, 1.0 / math.sqrt(D), np.float32)
    per_key = 10.0 / 64 / (scale * math.log2(math.e))      # score growth per key, before the scale
    q = 4.0 * u + 0.1 * rng.standard_normal((1, 2, L, D), dtype=np.float32)
    k = (per_key / 4.0) * np.arange(L, dtype=np.float32)[None, None, :, None] * u \
        + 0.1 * rng.standard_normal((1, 1, L, D), dtype=np.float32)
    v = rng.standard_normal((1, 1, L, D), dtype=np.float32)
    cast = W.bf16_bits_from_f32 if dtype == "bf16" else (lambda a: a.astype(np.float16))
    q, k, v = cast(q), cast(k), cast(v)
    want = ref.prefill(q, k, v, scale=scale, causal=causal)
    got = mi.attn_prefill(to_gpu(q), to_gpu(k), to_gpu(v), causal=causal, scale=scale)
    import torch
    torch.cuda.synchronize()
    check(to_f64(got), want, dtype, f"growing scores {dtype} D {D} causal {causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_running_max_keeps_moving(mi, ref, D, dtype):
    """Decode over a cache whose scores grow by about 10 (log2 units) per 64 positions:
    each key range's running max keeps moving past the lazy-rescale slack, and the
    partial states of the ranges differ by orders of magnitude before they are combined."""
    say(f"decode growing scores {dtype} D {D}")
    rng = np.random.default_rng(29)
    B, Hq, Hkv, L, scale = 4, 8, 2, 1000, 1.0 / math.sqrt(D)
    u = np.full(D, 1.0 / math.sqrt(D), np.float32)
    per_key = 10.0 / 64 / (scale * math.log2(math.e))
    q = 4.0 * u + 0.1 * rng.standard_normal((B, Hq, D), dtype=np.float32)
    k = (per_key / 4.0) * np.arange(L, dtype=np.float32)[None, None, :, None] * u \
        + 0.1 * rng.standard_normal((B, Hkv, L, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, L, D), dtype=np.float32)
    cast = W.bf16_bits_from_f32 if dtype == "bf16" else (lambda a: a.astype(np.float16))
    q, k, v = cast(q), cast(k), cast(v)
    want = ref.decode(q, k, v, kv_len=L, scale=scale, pos_offset=L - 1)
    got = mi.attn_decode(to_gpu(q), to_gpu(k), to_gpu(v), kv_len=L, pos_offset=L - 1, scale=scale)
    import torch
    torch.cuda.synchronize()
    check(to_f64(got), want, dtype, f"decode growing scores {dtype} D {D}")


# ---------------------------------------------------------------------------
# edge cases

def test_empty_calls(mi):
    import torch
    q = torch.empty((0, 4, 16, 64), dtype=torch.bfloat16, device="cuda")
    assert mi.attn_prefill(q, q, q).shape == q.shape
    q = torch.empty((2, 4, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((2, 4, 0, 64), dtype=torch.bfloat16, device="cuda")
    assert mi.attn_prefill(q, k, k).numel() == 0
    qd = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    kc = torch.empty((0, 4, 16, 64), dtype=torch.bfloat16, device="cuda")
    assert mi.attn_decode(qd, kc, kc).numel() == 0


def test_decode_all_items_empty(mi):
    import torch
    x = W.random_decode(3, 3, 8, 2, 64, 128, "bf16")
    lens = torch.zeros(3, dtype=torch.int32, device="cuda")
    out = mi.attn_decode(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), kv_len=64, kv_lens=lens)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_prefill_writes_only_its_output(mi, ref):
    """A canary after `out` in the same allocation stays untouched."""
    import torch
    x = W.random_prefill(5, 1, 4, 2, 200, 200, 128, "bf16")
    n = 1 * 4 * 200 * 128
    buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[:n].view(1, 4, 200, 128)
    mi.attn_prefill(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), out, causal=True)
    torch.cuda.synchronize()
    assert torch.all(buf[n:] == 7.0)
    want = ref.prefill(x["q"], x["k"], x["v"], scale=1 / math.sqrt(128), causal=True)
    check(to_f64(out), want, "bf16", "canary run")


def test_repeat_runs_are_bitwise_identical(mi):
    import torch
    x = W.random_prefill(9, 1, 8, 2, 512, 512, 128, "bf16")
    q, k, v = to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"])
    a = mi.attn_prefill(q, k, v, causal=True).clone()
    b = mi.attn_prefill(q, k, v, causal=True).clone()
    xd = W.random_decode(9, 8, 32, 8, 4096, 128, "bf16")
    qd, kd, vd = to_gpu(xd["q"]), to_gpu(xd["k"]), to_gpu(xd["v"])
    c = mi.attn_decode(qd, kd, vd).clone()
    d = mi.attn_decode(qd, kd, vd).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), d.view(torch.int16))


# ---------------------------------------------------------------------------
# the five named workloads at full size


@pytest.mark.parametrize("name", ["tiny_causal_f32", "bert_base_padded", "banded_w128_s8192", "causal_gqa_s4096",
                                  "causal_gqa_s4096_f16"])
def test_named_prefill_workload(mi, ref, name):
    """Every output row of the named workload against the oracle (the oracle runs on all
    host cores: the causal GQA workload is 137 GFLOP of fp64 work)."""
    import torch
    w = W.WORKLOADS[name]
    say(f"workload {name}")
    x = W.make_inputs(w)
    seq = x["seq_lens"]
    got = mi.attn_prefill(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), pos_offset=w.pos_offset,
                          seq_lens=None if seq is None else to_gpu(seq), window=w.window, causal=w.causal,
                          scale=w.attn_scale)
    torch.cuda.synchronize()
    g = to_f64(got)
    del got
    want = ref.prefill(x["q"], x["k"], x["v"], scale=w.attn_scale, causal=w.causal, pos_offset=w.pos_offset,
                       seq_lens=seq, window=w.window)
    if seq is not None:   # padded query rows are written as zeros
        for b in range(w.batch):
            assert np.all(g[b, :, max(0, int(seq[b]) - w.pos_offset):] == 0.0), "padded query rows must be zero"
    record(name, check(g, want, w.dtype, name))


@pytest.mark.parametrize("name", ["gqa_decode_kv8192", "gqa_decode_kv8192_f16"])
def test_named_decode_workload(mi, ref, name):
    import torch
    w = W.WORKLOADS[name]
    say(f"workload {name}")
    x = W.make_inputs(w)
    got = mi.attn_decode(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), kv_len=w.kv_len, pos_offset=w.pos_offset,
                         window=w.window, scale=w.attn_scale)
    torch.cuda.synchronize()
    want = ref.decode(x["q"], x["k"], x["v"], kv_len=w.kv_len, scale=w.attn_scale, pos_offset=w.pos_offset,
                      window=w.window)
    record(name, check(to_f64(got), want, w.dtype, name))
