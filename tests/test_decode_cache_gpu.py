"""GPU parity of the per-item-cache decode calls against the fp64 oracle.

attn_decode_per_cache attends each item's query over its own, separately allocated
head-major cache; attn_decode_append first writes the new token's K/V row into slot
cache_lens[b] of each item's cache and attends over the cache including it, in one
launch (ferrum-kernels `Backend`, Provided Methods: `flash_attention_batched_per_cache`,
`kv_cache_append_batched_per_cache`).  Outputs are compared element by element with the
tolerances of the other parity tests; the caches after an append are compared bit for
bit with the oracle's (a copy is exact).
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


def _nan(dtype):
    return W.BF16_NAN if dtype == "bf16" else np.float32(np.nan)


def _bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.itemsize == 2 else a.view(np.uint32)


def _host(t, dtype) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _items(rng_seed, B, Hq, Hkv, cap, D, dtype):
    rng = np.random.default_rng(rng_seed)
    q = W.draw(rng, (B, Hq, D), 1.0, dtype)
    kc = [W.draw(rng, (Hkv, cap, D), 1.0, dtype) for _ in range(B)]
    vc = [W.draw(rng, (Hkv, cap, D), 1.0, dtype) for _ in range(B)]
    kn = W.draw(rng, (B, Hkv, D), 1.0, dtype)
    vn = W.draw(rng, (B, Hkv, D), 1.0, dtype)
    return q, kc, vc, kn, vn


PER_ITEM_CASES = [
    # B, Hq, Hkv, capacity, D, lengths, window, dtype
    (4, 32, 8, 1024, 128, [1000, 1, 0, 1024], 0, "bf16"),
    (3, 16, 1, 700, 128, [699, 350, 2], 5, "bf16"),        # 16 query heads per kv head: two head groups
    (5, 8, 8, 300, 64, [300, 299, 150, 64, 1], 0, "bf16"),
    (3, 12, 4, 513, 32, [513, 100, 3], 64, "bf16"),
    (2, 4, 1, 300, 128, [300, 299], 17, "f32"),
    (3, 6, 2, 256, 64, [200, 50, 256], 0, "f32"),
    (64, 8, 8, 96, 64, [(37 * i) % 97 for i in range(64)], 0, "f32"),  # 512 units: one workgroup each
    (4, 32, 8, 1024, 128, [1000, 1, 0, 1024], 7, "f16"),
]


def _ids(c):
    return "x".join(map(str, c[:5])) + f"-W{c[6]}-{c[7]}"


@pytest.mark.parametrize("case", PER_ITEM_CASES, ids=_ids)
def test_decode_per_cache_parity(mi, ref, case):
    import torch
    B, Hq, Hkv, cap, D, lens, Wn, dt = case
    say(f"decode_per_cache case {case}")
    q, kc, vc, _, _ = _items(21, B, Hq, Hkv, cap, D, dt)
    lens = np.array(lens, np.int32)
    for b in range(B):   # slots at or past an item's length are never read
        kc[b][:, lens[b]:] = _nan(dt)
        vc[b][:, lens[b]:] = _nan(dt)
    scale = 1.0 / math.sqrt(D)
    want = ref.decode_per_cache(q, kc, vc, lens, scale=scale, window=Wn)
    # each item's caches in an allocation of their own
    kd, vd = [to_gpu(c) for c in kc], [to_gpu(c) for c in vc]
    got = mi.attn_decode_per_cache(to_gpu(q), kd, vd, to_gpu(lens), window=Wn, scale=scale)
    torch.cuda.synchronize()
    check(to_f64(got), want, dt, f"decode_per_cache {case}")


APPEND_CASES = [
    # B, Hq, Hkv, capacity, D, cache lengths (before the append), window, dtype
    (4, 32, 8, 1024, 128, [999, 0, 1023, 1024], 0, "bf16"),   # last slot; no room
    (3, 16, 1, 700, 128, [698, 349, -1], 5, "bf16"),
    (5, 8, 8, 300, 64, [299, 298, 149, 63, 0], 0, "bf16"),
    (3, 12, 4, 513, 32, [512, 99, 2], 64, "bf16"),
    (2, 4, 1, 300, 128, [299, 298], 17, "f32"),
    (3, 6, 2, 256, 64, [199, 49, 255], 0, "f32"),
    (64, 8, 8, 96, 64, [(37 * i) % 97 - 1 for i in range(64)], 0, "f32"),
    (4, 32, 8, 1024, 128, [999, 0, 1023, 1024], 0, "f16"),
    (3, 12, 4, 513, 64, [512, 99, 2], 64, "f16"),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=_ids)
def test_decode_append_parity(mi, ref, case):
    import torch
    B, Hq, Hkv, cap, D, lens, Wn, dt = case
    say(f"decode_append case {case}")
    q, kc, vc, kn, vn = _items(22, B, Hq, Hkv, cap, D, dt)
    lens = np.array(lens, np.int32)
    for b in range(B):   # the slot written and everything after it: NaN before the call
        lo = min(max(int(lens[b]), 0), cap)
        kc[b][:, lo:] = _nan(dt)
        vc[b][:, lo:] = _nan(dt)
    scale = 1.0 / math.sqrt(D)
    want, k_after, v_after = ref.decode_append(q, kn, vn, kc, vc, lens, scale=scale, window=Wn)
    kd, vd = [to_gpu(c) for c in kc], [to_gpu(c) for c in vc]
    got = mi.attn_decode_append(to_gpu(q), to_gpu(kn), to_gpu(vn), kd, vd, to_gpu(lens), window=Wn, scale=scale)
    torch.cuda.synchronize()
    check(to_f64(got), want, dt, f"decode_append {case}")
    for b in range(B):
        assert np.array_equal(_bits(_host(kd[b], dt)), _bits(k_after[b])), f"K cache of item {b} after the append"
        assert np.array_equal(_bits(_host(vd[b], dt)), _bits(v_after[b])), f"V cache of item {b} after the append"


def test_decode_append_two_steps(mi, ref):
    """Two decode steps in a row: the second attends over the row the first appended."""
    import torch
    B, Hq, Hkv, cap, D, dt = 3, 8, 2, 200, 128, "bf16"
    say("decode_append two steps")
    q, kc, vc, kn, vn = _items(23, B, Hq, Hkv, cap, D, dt)
    q2, _, _, kn2, vn2 = _items(24, B, Hq, Hkv, cap, D, dt)
    lens = np.array([10, 0, 198], np.int32)
    scale = 1.0 / math.sqrt(D)
    w1, k1, v1 = ref.decode_append(q, kn, vn, kc, vc, lens, scale=scale)
    w2, k2, v2 = ref.decode_append(q2, kn2, vn2, k1, v1, lens + 1, scale=scale)
    table_k = mi.CacheTable([to_gpu(c) for c in kc])
    table_v = mi.CacheTable([to_gpu(c) for c in vc])
    g1 = mi.attn_decode_append(to_gpu(q), to_gpu(kn), to_gpu(vn), table_k, table_v, to_gpu(lens), scale=scale)
    g2 = mi.attn_decode_append(to_gpu(q2), to_gpu(kn2), to_gpu(vn2), table_k, table_v, to_gpu(lens + 1),
                               scale=scale)
    torch.cuda.synchronize()
    check(to_f64(g1), w1, dt, "step 1")
    check(to_f64(g2), w2, dt, "step 2")
    for b in range(B):
        assert np.array_equal(_host(table_k.caches[b], dt), k2[b])
        assert np.array_equal(_host(table_v.caches[b], dt), v2[b])


def test_decode_append_matches_plain_decode(mi):
    """Append + attend equals writing the row on the host and running attn_decode over
    the stacked caches with kv_lens = cache_lens + 1 (the kernels share their arithmetic,
    so the outputs agree bit for bit)."""
    import torch
    B, Hq, Hkv, cap, D, dt = 4, 32, 8, 512, 128, "bf16"
    say("decode_append vs attn_decode")
    q, kc, vc, kn, vn = _items(25, B, Hq, Hkv, cap, D, dt)
    lens = np.array([511, 0, 300, 17], np.int32)
    K, V = np.stack(kc), np.stack(vc)
    Kw, Vw = K.copy(), V.copy()
    for b in range(B):
        Kw[b, :, lens[b]] = kn[b]
        Vw[b, :, lens[b]] = vn[b]
    plain = mi.attn_decode(to_gpu(q), to_gpu(Kw), to_gpu(Vw), kv_len=cap, kv_lens=to_gpu(lens + 1))
    Kd, Vd = to_gpu(K), to_gpu(V)
    fused = mi.attn_decode_append(to_gpu(q), to_gpu(kn), to_gpu(vn), Kd, Vd, to_gpu(lens))
    torch.cuda.synchronize()
    assert torch.equal(plain, fused)
    assert np.array_equal(_host(Kd, dt), Kw) and np.array_equal(_host(Vd, dt), Vw)


def test_named_decode_append_workload(mi, ref):
    """The 64-item, 8192-slot GQA decode with the append, in the benchmark's launch
    configuration (a stacked cache tensor addressed through a cache table)."""
    import torch
    w = W.WORKLOADS["gqa_decode_append_kv8192"]
    say("workload gqa_decode_append_kv8192")
    x = W.make_inputs(w)
    kd, vd = to_gpu(x["k"]), to_gpu(x["v"])
    got = mi.attn_decode_append(to_gpu(x["q"]), to_gpu(x["k_new"]), to_gpu(x["v_new"]), mi.CacheTable(kd),
                                mi.CacheTable(vd), to_gpu(x["cache_lens"]), window=w.window, scale=w.attn_scale)
    torch.cuda.synchronize()
    want, k_after, v_after = ref.decode_append(x["q"], x["k_new"], x["v_new"], list(x["k"]), list(x["v"]),
                                               x["cache_lens"], scale=w.attn_scale, window=w.window)
    record(w.name, check(to_f64(got), want, w.dtype, w.name))
    assert np.array_equal(_host(kd, w.dtype), np.stack(k_after)), "K caches after the append"
    assert np.array_equal(_host(vd, w.dtype), np.stack(v_after)), "V caches after the append"


QKV_CASES = [
    # B, Hq, Hkv, capacity, D, cache lengths (before the append), window, dtype
    (4, 32, 8, 1024, 128, [999, 0, 1023, 1024], 0, "bf16"),
    (3, 12, 4, 513, 64, [512, 99, 2], 64, "f16"),
    (3, 6, 2, 256, 32, [199, 49, 255], 0, "f32"),
]


@pytest.mark.parametrize("case", QKV_CASES, ids=_ids)
def test_decode_append_qkv(mi, ref, case):
    """The new token's q, k and v read from one fused row per item [q heads | k heads | v
    heads] (ferrum-kernels `Backend` page, `split_qkv` layout): against the oracle on the
    split tensors, and bit for bit against attn_decode_append on them (outputs and caches)."""
    import torch
    B, Hq, Hkv, cap, D, lens, Wn, dt = case
    say(f"decode_append_qkv case {case}")
    q, kc, vc, kn, vn = _items(26, B, Hq, Hkv, cap, D, dt)
    lens = np.array(lens, np.int32)
    qkv = np.concatenate([q, kn, vn], axis=1)   # [B, Hq + 2 Hkv, D]
    scale = 1.0 / math.sqrt(D)
    want, k_after, v_after = ref.decode_append(q, kn, vn, kc, vc, lens, scale=scale, window=Wn)
    kd, vd = [to_gpu(c) for c in kc], [to_gpu(c) for c in vc]
    got = mi.attn_decode_append_qkv(to_gpu(qkv), kd, vd, to_gpu(lens), window=Wn, scale=scale)
    kd2, vd2 = [to_gpu(c) for c in kc], [to_gpu(c) for c in vc]
    split = mi.attn_decode_append(to_gpu(q), to_gpu(kn), to_gpu(vn), kd2, vd2, to_gpu(lens), window=Wn, scale=scale)
    torch.cuda.synchronize()
    record(f"decode_append_qkv {case[:5]}", check(to_f64(got), want, dt, f"decode_append_qkv {case}"))
    assert torch.equal(got, split), "fused-row and split calls must agree bit for bit"
    for b in range(B):
        assert np.array_equal(_bits(_host(kd[b], dt)), _bits(k_after[b])), f"K cache of item {b} after the append"
        assert np.array_equal(_bits(_host(vd[b], dt)), _bits(v_after[b])), f"V cache of item {b} after the append"
