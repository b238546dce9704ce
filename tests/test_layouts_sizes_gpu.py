"""GPU parity of the token-major prefill, and of the largest sizes the calls take.

attn_prefill_token_major reads q [B, Lq, Hq, D] and k, v [B, Lk, Hkv, D] and writes out
[B, Lq, Hq, D] (the layout around the pages' head-major attention: ferrum-kernels
`Backend`, `transpose_head_to_token`; ripvec-core `Driver`, `attn_reshape`).  Its rows are
computed exactly as the head-major launch computes them, so the two agree bit for bit.

The size cases run the longest cache and sequence and the largest grid of the tests,
checked on sampled rows or items.
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


TM_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, causal, P, seq_lens, W, dtype
    (1, 8, 2, 257, 257, 128, True, 0, None, 0, "bf16"),
    (2, 4, 4, 333, 333, 64, False, 0, [333, 100], 128, "bf16"),
    (2, 6, 3, 130, 200, 32, True, 70, None, 0, "bf16"),
    (1, 4, 2, 300, 300, 64, True, 0, None, 0, "f16"),
    (2, 2, 1, 70, 90, 128, False, 20, [85, 40], 9, "f32"),
    # padded items at head dims 128 and 32: whole waves and q-tiles of rows that see no key
    (2, 8, 2, 300, 300, 128, False, 0, [300, 129], 0, "bf16"),
    (3, 4, 2, 200, 200, 32, True, 0, [200, 70, 1], 0, "f16"),
]


@pytest.mark.parametrize("case", TM_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-c{int(c[6])}-W{c[9]}-{c[10]}")
def test_token_major_parity(mi, ref, case):
    import torch
    B, Hq, Hkv, Lq, Lk, D, causal, P, sl, Wn, dt = case
    say(f"token-major case {case}")
    rng = np.random.default_rng(41)
    q = W.draw(rng, (B, Lq, Hq, D), 1.0, dt)
    k = W.draw(rng, (B, Lk, Hkv, D), 1.0, dt)
    v = W.draw(rng, (B, Lk, Hkv, D), 1.0, dt)
    seq = None if sl is None else np.array(sl, np.int32)
    if seq is not None:
        # NaN in every query row that sees no key and every key/value row past the valid
        # ones: such inputs must not reach any output (rows that see no key are written as 0)
        nan = W.BF16_NAN if dt == "bf16" else np.float32(np.nan)
        for b in range(B):
            q[b, max(min(int(seq[b]), Lk) - P, 0):] = nan
            k[b, max(min(int(seq[b]), Lk), 0):] = nan
            v[b, max(min(int(seq[b]), Lk), 0):] = nan
    scale = 1.0 / math.sqrt(D)
    kw = dict(pos_offset=P, window=Wn, causal=causal, scale=scale)
    want = ref.prefill_token_major(q, k, v, seq_lens=seq, **kw)
    sd = None if seq is None else to_gpu(seq)
    got = mi.attn_prefill_token_major(to_gpu(q), to_gpu(k), to_gpu(v), seq_lens=sd, **kw)
    # the head-major launch on the same values
    hm = mi.attn_prefill(to_gpu(np.ascontiguousarray(q.transpose(0, 2, 1, 3))),
                         to_gpu(np.ascontiguousarray(k.transpose(0, 2, 1, 3))),
                         to_gpu(np.ascontiguousarray(v.transpose(0, 2, 1, 3))), seq_lens=sd, **kw)
    torch.cuda.synchronize()
    g = to_f64(got)
    if seq is not None:
        for b in range(B):
            assert np.all(g[b, max(min(int(seq[b]), Lk) - P, 0):] == 0.0), "rows that see no key must be zero"
    check(g, want, dt, f"token-major {case}")
    assert torch.equal(got, hm.transpose(1, 2).contiguous()), "token-major and head-major launches differ"


def test_named_token_major_workload(mi, ref):
    """The causal GQA prefill (1 x 4096 tokens, 32/8 heads, head_dim 128) on token-major
    tensors, in the benchmark's launch configuration: every output row against the oracle."""
    import torch
    w = W.WORKLOADS["causal_gqa_s4096_token_major"]
    say("workload causal_gqa_s4096_token_major")
    x = W.make_inputs(w)
    got = mi.attn_prefill_token_major(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), causal=w.causal,
                                      scale=w.attn_scale)
    torch.cuda.synchronize()
    g = to_f64(got)
    want = ref.prefill_token_major(x["q"], x["k"], x["v"], scale=w.attn_scale, causal=True)
    record(w.name, check(g, want, w.dtype, w.name))


def test_long_decode_cache(mi, ref):
    """One item, one kv head, 262144 cached positions (head_dim 128, bf16): the split plan
    cuts the range into many splits; checked against the oracle."""
    import torch
    B, Hq, Hkv, cap, D = 1, 8, 1, 262144, 128
    say("long decode: capacity 262144")
    x = W.random_decode(51, B, Hq, Hkv, cap, D, "bf16")
    lens = np.array([cap - 5], np.int32)
    scale = 1.0 / math.sqrt(D)
    want = ref.decode(x["q"], x["k"], x["v"], kv_len=cap, scale=scale, kv_lens=lens)
    got = mi.attn_decode(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), kv_len=cap, kv_lens=to_gpu(lens),
                         scale=scale)
    torch.cuda.synchronize()
    check(to_f64(got), want, "bf16", "long decode")


def test_long_prefill_sampled_rows(mi, ref):
    """32768 tokens, causal, GQA 4/2, head_dim 64 (bf16): sampled rows, including the first
    and last, against the oracle."""
    import torch
    B, Hq, Hkv, L, D = 1, 4, 2, 32768, 64
    say("long prefill: 32768 tokens")
    x = W.random_prefill(52, B, Hq, Hkv, L, L, D, "bf16")
    scale = 1.0 / math.sqrt(D)
    got = mi.attn_prefill(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), causal=True, scale=scale)
    torch.cuda.synchronize()
    g = to_f64(got)
    rng = np.random.default_rng(3)
    rows = [(0, h, i) for h in range(Hq) for i in (0, L - 1)]
    rows += [(0, int(h), int(i)) for h, i in zip(rng.integers(0, Hq, 60), rng.integers(0, L, 60))]
    rows = np.array(rows, np.int32)
    want = ref.prefill(x["q"], x["k"], x["v"], scale=scale, causal=True, rows=rows)
    check(g[rows[:, 0], rows[:, 1], rows[:, 2]], want, "bf16", "long prefill rows")


def test_many_items(mi, ref):
    """16384 items of 4 heads: 65536 q-tiles, so the head-dim-64 kernel's persistent grid
    grows past the resident workgroups to keep every list within 64 q-tiles; padded
    lengths.  The output starts as NaN: every element must be written (rows past an
    item's length as zeros); sampled items against the oracle."""
    import torch
    B, Hq, Hkv, L, D = 16384, 4, 1, 64, 64
    say("many items: 16384")
    x = W.random_prefill(53, B, Hq, Hkv, L, L, D, "bf16", seq_len_range=(1, 64))
    scale = 1.0 / math.sqrt(D)
    out = torch.full((B, Hq, L, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    mi.attn_prefill(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), out, seq_lens=to_gpu(x["seq_lens"]),
                    scale=scale)
    torch.cuda.synchronize()
    g = to_f64(out)
    assert np.all(np.isfinite(g)), "a q-tile of the output was not written"
    lens = x["seq_lens"]
    assert all(np.all(g[b, :, int(lens[b]):] == 0.0) for b in range(0, B, 97)), "padded rows must be zero"
    for b in (0, 1, 8191, 16382, 16383):
        want = ref.prefill(x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], scale=scale,
                           seq_lens=x["seq_lens"][b:b + 1])
        check(g[b:b + 1], want, "bf16", f"item {b}")
