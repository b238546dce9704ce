"""GPU parity of attn_prefill_varlen (unpadded, token-major batches) against the fp64 oracle.

Items of ragged lengths are concatenated token-major, q/out [tokens, q_heads, D] and
k/v [tokens, kv_heads, D], with cu_seqlens boundaries (ripvec-core `Driver`,
`prepare_batch_unpadded`).  Element by element, bf16: |gpu - ref| <= 2e-2 + 1e-2 |ref|,
fp32: max abs 1e-4.  The unpadded and padded launches compute every row the same way,
so on the BERT-shaped batch they must agree bit for bit.
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


def _batch(seed, lens, Hq, Hkv, D, dtype):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    q = W.draw(rng, (T, Hq, D), 1.0, dtype)
    k = W.draw(rng, (T, Hkv, D), 1.0, dtype)
    v = W.draw(rng, (T, Hkv, D), 1.0, dtype)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, cu


VARLEN_CASES = [
    # item lengths, Hq, Hkv, D, causal, window, dtype
    ([300, 0, 17, 513], 4, 4, 64, False, 0, "bf16"),
    ([257, 1, 300], 8, 2, 128, True, 0, "bf16"),
    ([600, 129], 4, 2, 128, False, 200, "bf16"),
    ([200, 64, 1], 6, 3, 32, False, 0, "bf16"),
    ([333, 2], 4, 4, 64, True, 128, "bf16"),
    ([520, 300, 280, 10], 8, 2, 128, True, 0, "bf16"),   # 8 (item, kv head) units: XCD-grouped order
    ([150, 99], 4, 2, 64, True, 0, "f32"),
    ([65, 130], 2, 1, 128, False, 9, "f32"),
    ([100, 33, 0, 7], 4, 4, 32, True, 16, "f32"),
    ([300, 0, 17, 513], 4, 4, 64, False, 0, "f16"),
    ([257, 1, 300], 8, 2, 128, True, 0, "f16"),
    # narrow bands over unpadded items at head dims 32/64 (bidirectional and causal windows)
    ([1000, 5, 700, 129], 4, 2, 64, False, 128, "bf16"),
    ([900, 33], 2, 2, 32, True, 64, "f16"),
]


@pytest.mark.parametrize("case", VARLEN_CASES,
                         ids=lambda c: "-".join(map(str, c[0])) + f"-{c[1]}x{c[2]}x{c[3]}-c{int(c[4])}-W{c[5]}-{c[6]}")
def test_prefill_varlen_parity(mi, ref, case):
    import torch
    lens, Hq, Hkv, D, causal, Wn, dt = case
    say(f"varlen case {case}")
    q, k, v, cu = _batch(31, lens, Hq, Hkv, D, dt)
    scale = 1.0 / math.sqrt(D)
    want = ref.prefill_varlen(q, k, v, cu, scale=scale, causal=causal, window=Wn)
    got = mi.attn_prefill_varlen(to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(cu), max(lens), window=Wn, causal=causal,
                                 scale=scale)
    torch.cuda.synchronize()
    check(to_f64(got), want, dt, f"varlen {case}")


def test_prefill_varlen_max_seqlen_cut(mi, ref):
    """An item longer than max_seqlen is computed as its first max_seqlen tokens; its
    later rows of out are left as they were."""
    import torch
    lens, Hq, Hkv, D, dt = [300, 50], 4, 2, 64, "bf16"
    say("varlen max_seqlen cut")
    q, k, v, cu = _batch(32, lens, Hq, Hkv, D, dt)
    out = torch.full((sum(lens), Hq, D), 7.0, dtype=torch.bfloat16, device="cuda")
    mi.attn_prefill_varlen(to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(cu), 200, out, causal=False)
    torch.cuda.synchronize()
    g = to_f64(out)
    scale = 1.0 / math.sqrt(D)
    first = ref.prefill_varlen(q[:200], k[:200], v[:200], np.array([0, 200], np.int32), scale=scale)
    second = ref.prefill_varlen(q[300:], k[300:], v[300:], np.array([0, 50], np.int32), scale=scale)
    check(g[:200], first, dt, "first 200 tokens of the long item")
    assert np.all(g[200:300] == 7.0), "rows past max_seqlen were written"
    check(g[300:], second, dt, "second item")


def test_prefill_varlen_empty_calls(mi):
    import torch
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16, device="cuda")
    cu0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = mi.attn_prefill_varlen(q, q, q, cu0, 0)
    cu = torch.tensor([0, 0, 0], dtype=torch.int32, device="cuda")
    out2 = mi.attn_prefill_varlen(q, q, q, cu, 0)
    torch.cuda.synchronize()
    assert out.shape == q.shape and out2.shape == q.shape


def test_bert_varlen_matches_padded_launch(mi, ref):
    """The BERT-shaped batch, unpadded, in the benchmark's launch configuration: every row
    against the oracle, and every row bit-identical to the padded-layout launch."""
    import torch
    w = W.WORKLOADS["bert_base_varlen"]
    say("workload bert_base_varlen")
    x = W.make_inputs(w)
    lens, cu = x["seq_lens"], x["cu_seqlens"]
    got = mi.attn_prefill_varlen(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), to_gpu(cu), int(lens.max()),
                                 causal=w.causal, window=w.window, scale=w.attn_scale)
    # the same tokens in the padded head-major layout [B, H, 512, D]
    B, H, D, L = w.batch, w.q_heads, w.head_dim, w.q_len
    pad = {}
    for name in ("q", "k", "v"):
        a = np.zeros((B, H, L, D), np.uint16)
        for b in range(B):
            a[b, :, :lens[b]] = x[name][cu[b]:cu[b + 1]].transpose(1, 0, 2)
        pad[name] = a
    padded = mi.attn_prefill(to_gpu(pad["q"]), to_gpu(pad["k"]), to_gpu(pad["v"]), seq_lens=to_gpu(lens),
                             causal=w.causal, window=w.window, scale=w.attn_scale)
    torch.cuda.synchronize()
    g = got.view(torch.int16).cpu().numpy()
    p = padded.view(torch.int16).cpu().numpy()
    for b in range(B):
        assert np.array_equal(g[cu[b]:cu[b + 1]], p[b, :, :lens[b]].transpose(1, 0, 2)), f"item {b}"
    want = ref.prefill_varlen(x["q"], x["k"], x["v"], cu, scale=w.attn_scale, causal=w.causal, window=w.window)
    record(w.name, check(to_f64(got), want, w.dtype, w.name))
