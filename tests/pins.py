"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin is a function ``pin_x(oracle)`` that raises AssertionError when the oracle
disagrees with what the pages and the mathematics fix.  They are collected in
``PINS`` so that ``test_oracle_pins`` can run them on the real oracle and
``test_oracle_mutants`` can show that each planted mistake fails at least one of them.

Sources of truth used here (none of them calls the oracle's own arithmetic):
  * hand-worked examples with exact answers (``golden/hand_worked.json``);
  * a brute-force transcription of the definition in pure-Python loops (``brute.py``);
  * torch's CPU ``scaled_dot_product_attention`` in float64 (a library routine that
    the unmasked/masked case reduces to);
  * closed forms: constant V rows, causal row 0, a single key, two keys (sigmoid),
    scale 0 (plain mean over the key set), one-hot V (exposes the weights and their
    count), windows at least as long as the sequence;
  * invariances: NaN-poisoned padding, GQA == MHA with repeated K/V, chunked prefill,
    joint permutation of K and V rows, decode == per-item decode.
"""
from __future__ import annotations

import json
import math
from pathlib import Path

import numpy as np

import brute
from workloads import BF16_NAN, bf16_bits_from_f32, draw, f32_from_bf16_bits

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


def _f64(a):
    return f32_from_bf16_bits(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# hand-worked examples

def _parse(x):
    if isinstance(x, list):
        return [_parse(e) for e in x]
    if isinstance(x, str) and x.startswith("ln(") and x.endswith(")"):
        return float(np.float32(math.log(float(x[3:-1]))))
    return float(x)


def pin_hand_worked(oracle):
    cases = json.loads((GOLDEN / "hand_worked.json").read_text())["cases"]
    for c in cases:
        q = np.array(_parse(c["q"]), np.float32)
        k = np.array(_parse(c["k"]), np.float32)
        v = np.array(_parse(c["v"]), np.float32)
        exp = np.array(c["expected"], np.float64)
        if c["kind"] == "prefill":
            got = oracle.prefill(q, k, v, scale=c["scale"], causal=c["causal"], pos_offset=c["pos_offset"],
                                 seq_lens=c["seq_lens"], window=c["window"])
        else:
            got = oracle.decode(q, k, v, kv_len=c["kv_len"], scale=c["scale"], pos_offset=c["pos_offset"],
                                kv_lens=c["kv_lens"], window=c["window"])
        tol = 1e-6 * max(1.0, float(np.max(np.abs(exp))))
        _close(got, exp, tol, c["name"])


# ---------------------------------------------------------------------------
# brute force on tiny shapes

_TINY = [
    # (B, Hq, Hkv, Lq, Lk, D, causal, P, seq_lens, window, dtype)
    (1, 1, 1, 5, 5, 4, True, 0, None, 0, "f32"),
    (2, 2, 2, 4, 6, 3, False, 0, [6, 3], 0, "f32"),
    (1, 4, 1, 3, 7, 4, True, 4, None, 0, "bf16"),
    (2, 4, 2, 6, 6, 2, False, 0, [0, 9], 3, "f32"),
    (1, 2, 1, 7, 7, 3, False, 0, None, 4, "bf16"),
    (1, 2, 2, 5, 8, 2, True, 3, [7], 3, "f32"),
    (1, 3, 3, 6, 6, 2, True, 0, None, 2, "f32"),
    (2, 2, 1, 3, 5, 5, True, 2, [4, 5], 0, "bf16"),
]


def pin_brute_force(oracle):
    for n, (B, Hq, Hkv, Lq, Lk, D, causal, P, sl, W, dt) in enumerate(_TINY):
        rng = _rng(100 + n)
        q = draw(rng, (B, Hq, Lq, D), 1.0, dt)
        k = draw(rng, (B, Hkv, Lk, D), 1.0, dt)
        v = draw(rng, (B, Hkv, Lk, D), 1.0, dt)
        scale = 1.0 / math.sqrt(D) * (1.0 + 0.25 * n)
        got = oracle.prefill(q, k, v, scale=scale, causal=causal, pos_offset=P, seq_lens=sl, window=W)
        ref = brute.attention(q, k, v, scale=scale, causal=causal, pos_offset=P, seq_lens=sl, window=W)
        _close(got, ref, 1e-12, f"tiny case {n}")


_TINY_DECODE = [
    # (B, Hq, Hkv, cap, kv_len, D, P, kv_lens, window)
    (2, 4, 2, 6, 5, 3, 4, None, 0),
    (3, 2, 1, 7, 7, 4, 0, [7, 1, 4], 0),
    (3, 4, 1, 8, 6, 2, 0, [6, 0, 3], 2),
    (1, 2, 2, 5, 5, 3, 2, None, 3),
]


def pin_brute_force_decode(oracle):
    for n, (B, Hq, Hkv, cap, L, D, P, kl, W) in enumerate(_TINY_DECODE):
        rng = _rng(200 + n)
        q = draw(rng, (B, Hq, D), 1.0, "f32")
        k = draw(rng, (B, Hkv, cap, D), 1.0, "f32")
        v = draw(rng, (B, Hkv, cap, D), 1.0, "f32")
        scale = 0.7 + 0.1 * n
        got = oracle.decode(q, k, v, kv_len=L, scale=scale, pos_offset=P, kv_lens=kl, window=W)
        ref = brute.decode(q, k, v, kv_len=L, scale=scale, pos_offset=P, kv_lens=kl, window=W)
        _close(got, ref, 1e-12, f"tiny decode case {n}")


# ---------------------------------------------------------------------------
# library cross-check

def pin_torch_sdpa(oracle):
    import torch
    import torch.nn.functional as F

    cases = [
        # (B, Hq, Hkv, Lq, Lk, D, causal, P, seq_lens, window)
        (2, 4, 2, 37, 37, 16, True, 0, None, 0),
        (2, 3, 3, 29, 29, 8, False, 0, [29, 11], 0),
        (1, 4, 1, 20, 45, 8, True, 25, None, 9),
        (1, 2, 2, 40, 40, 8, False, 0, None, 13),
    ]
    for n, (B, Hq, Hkv, Lq, Lk, D, causal, P, sl, W) in enumerate(cases):
        rng = _rng(300 + n)
        q, k, v = (draw(rng, s, 1.0, "bf16") for s in ((B, Hq, Lq, D), (B, Hkv, Lk, D), (B, Hkv, Lk, D)))
        scale = 1.0 / math.sqrt(D)
        got = oracle.prefill(q, k, v, scale=scale, causal=causal, pos_offset=P, seq_lens=sl, window=W)
        mask = np.zeros((B, 1, Lq, Lk), bool)
        for b in range(B):
            valid = Lk if sl is None else sl[b]
            for i in range(Lq):
                for j in brute.key_set(P + i, valid, causal, W):
                    mask[b, 0, i, j] = True
        tq, tk, tv = (torch.from_numpy(_f64(x)) for x in (q, k, v))
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=scale,
                                             enable_gqa=True).numpy()
        live = np.broadcast_to(mask.any(axis=-1)[..., None], ref.shape)
        _close(got[live], ref[live], 1e-12, f"sdpa case {n}")
        assert np.all(got[~live] == 0.0), f"sdpa case {n}: rows with no keys must be 0"


# ---------------------------------------------------------------------------
# closed forms

def pin_constant_v(oracle):
    """Every V row equal to c => every row with a key is exactly c (weights sum to 1)."""
    rng = _rng(400)
    B, Hq, Hkv, L, D = 2, 4, 2, 24, 8
    q = draw(rng, (B, Hq, L, D), 1.0, "f32")
    k = draw(rng, (B, Hkv, L, D), 1.0, "f32")
    c = np.arange(1, D + 1, dtype=np.float32) * np.float32(0.25) - np.float32(1.0)
    v = np.broadcast_to(c, (B, Hkv, L, D)).copy()
    for causal, W, sl in ((True, 0, None), (False, 5, [24, 10]), (True, 4, [15, 24])):
        out = oracle.prefill(q, k, v, scale=0.3, causal=causal, seq_lens=sl, window=W)
        for b in range(B):
            valid = L if sl is None else sl[b]
            _close(out[b, :, :valid], np.broadcast_to(c, out[b, :, :valid].shape), 1e-14, "constant V")
            assert np.all(out[b, :, valid:] == 0.0), "padded rows must be 0"


def pin_causal_row0(oracle):
    """Causal, position 0: the only key is key 0, so the output is V row 0 exactly."""
    rng = _rng(401)
    q = draw(rng, (2, 4, 9, 16), 1.0, "bf16")
    k = draw(rng, (2, 2, 9, 16), 1.0, "bf16")
    v = draw(rng, (2, 2, 9, 16), 1.0, "bf16")
    out = oracle.prefill(q, k, v, scale=0.25, causal=True)
    vf = _f64(v)
    for h in range(4):
        _close(out[:, h, 0], vf[:, h // 2, 0], 0.0, "causal row 0")


def pin_single_key(oracle):
    """One key: every row with a key returns that key's V row, whatever the scores."""
    rng = _rng(402)
    q = draw(rng, (1, 2, 1, 8), 1.0, "f32")
    k = draw(rng, (1, 2, 1, 8), 1.0, "f32")
    v = draw(rng, (1, 2, 1, 8), 1.0, "f32")
    for causal in (False, True):
        out = oracle.prefill(q, k, v, scale=3.0, causal=causal)
        _close(out[0, :, 0], v[0, :, 0].astype(np.float64), 0.0, "single key")


def pin_two_keys_sigmoid(oracle):
    """Scores (a, b) by construction => weight of key 0 is 1/(1+exp(b-a)); one-hot V exposes it."""
    a, b = np.float32(0.8125), np.float32(-1.375)
    for scale in (1.0, 0.5, 2.0):
        q = np.zeros((1, 1, 1, 4), np.float32)
        q[..., 0] = 1.0
        k = np.zeros((1, 1, 2, 4), np.float32)
        k[0, 0, 0, 0], k[0, 0, 1, 0] = a, b
        k[0, 0, :, 1] = 3.0  # orthogonal to q: must not matter
        v = np.zeros((1, 1, 2, 4), np.float32)
        v[0, 0, 0, 2], v[0, 0, 1, 3] = 1.0, 1.0
        out = oracle.prefill(q, k, v, scale=scale, causal=False)[0, 0, 0]
        w0 = 1.0 / (1.0 + math.exp(scale * (float(b) - float(a))))
        _close(out, [0.0, 0.0, w0, 1.0 - w0], 1e-15, f"two keys, scale {scale}")


def pin_scale_zero_mean(oracle):
    """scale 0 => uniform weights => the output is the plain mean of V over the key set."""
    rng = _rng(403)
    B, H, L, D = 1, 2, 20, 4
    q = draw(rng, (B, H, L, D), 1.0, "f32")
    k = draw(rng, (B, H, L, D), 1.0, "f32")
    v = draw(rng, (B, H, L, D), 1.0, "f32")
    vf = v.astype(np.float64)
    for causal, W in ((True, 0), (True, 6), (False, 7), (False, 0)):
        out = oracle.prefill(q, k, v, scale=0.0, causal=causal, window=W)
        for i in range(L):
            if causal:
                lo, hi = (0 if W == 0 else max(0, i - W + 1)), i
            else:
                lo, hi = (0, L - 1) if W == 0 else (max(0, i - W // 2), min(L - 1, i + W // 2))
            _close(out[0, :, i], vf[0, :, lo:hi + 1].mean(axis=1), 1e-14, f"mean, causal={causal} W={W} row {i}")


def _count_closed_form(p, valid, causal, W):
    if p >= valid:
        return 0
    if causal:
        hi = p
        lo = 0 if W == 0 else max(0, p - W + 1)
    else:
        hi = valid - 1 if W == 0 else min(valid - 1, p + W // 2)
        lo = 0 if W == 0 else max(0, p - W // 2)
    return max(0, hi - lo + 1)


def pin_key_counts_one_hot(oracle):
    """V = identity exposes the weights: each row's output is its weight vector.  Its
    support must have the closed-form size and its entries must sum to 1."""
    L = 16
    rng = _rng(404)
    q = draw(rng, (2, 2, 12, L), 0.5, "f32")
    k = draw(rng, (2, 2, L, L), 0.5, "f32")
    v = np.broadcast_to(np.eye(L, dtype=np.float32), (2, 2, L, L)).copy()
    for causal, W, P, sl in ((True, 0, 4, [16, 9]), (True, 5, 3, None), (False, 6, 0, [13, 16]),
                             (False, 7, 2, None), (False, 0, 0, [1, 16])):
        out = oracle.prefill(q, k, v, scale=0.6, causal=causal, pos_offset=P, seq_lens=sl, window=W)
        for b in range(2):
            valid = L if sl is None else sl[b]
            for i in range(12):
                want = _count_closed_form(P + i, valid, causal, W)
                for h in range(2):
                    w = out[b, h, i]
                    assert int(np.count_nonzero(w)) == want, \
                        f"row ({b},{h},{i}) causal={causal} W={W}: {np.count_nonzero(w)} keys, want {want}"
                    if want:
                        assert abs(w.sum() - 1.0) < 1e-12, "weights must sum to 1"
                        assert np.all(w >= 0)


def pin_probs_entry(oracle):
    """The inspection entry agrees with the closed-form support and sums to 1."""
    rng = _rng(405)
    q = draw(rng, (1, 2, 10, 8), 1.0, "bf16")
    k = draw(rng, (1, 1, 30, 8), 1.0, "bf16")
    v = draw(rng, (1, 1, 30, 8), 1.0, "bf16")
    for i in range(10):
        probs, row, n = oracle.prefill_probs(q, k, v, 0, 1, i, scale=0.4, causal=True, pos_offset=20, window=7)
        assert n == _count_closed_form(20 + i, 30, True, 7)
        assert abs(probs.sum() - 1.0) < 1e-12
        _close(row, probs @ _f64(v)[0, 0], 1e-13, "probs reproduce the row")


def pin_window_covers_sequence(oracle):
    """A causal window >= kv_len is full causal attention; a bidirectional window >= 2*kv_len
    is full attention; a bidirectional window of exactly kv_len is not."""
    rng = _rng(406)
    L = 11
    q = draw(rng, (1, 2, L, 8), 1.0, "f32")
    k = draw(rng, (1, 2, L, 8), 1.0, "f32")
    v = draw(rng, (1, 2, L, 8), 1.0, "f32")
    full_c = oracle.prefill(q, k, v, scale=0.5, causal=True)
    full_b = oracle.prefill(q, k, v, scale=0.5, causal=False)
    _close(oracle.prefill(q, k, v, scale=0.5, causal=True, window=L), full_c, 0.0, "causal window = L")
    _close(oracle.prefill(q, k, v, scale=0.5, causal=True, window=5 * L), full_c, 0.0, "causal window >> L")
    _close(oracle.prefill(q, k, v, scale=0.5, causal=False, window=2 * L), full_b, 0.0, "bidir window 2L")
    assert np.max(np.abs(oracle.prefill(q, k, v, scale=0.5, causal=False, window=L) - full_b)) > 1e-6, \
        "a bidirectional window of kv_len must still cut the far corners"


# ---------------------------------------------------------------------------
# invariances

def pin_padding_ignored(oracle):
    """NaN in every padded key/value position leaves valid rows bit-identical, padded rows 0,
    and valid rows equal to running each item on its truncated sequence."""
    rng = _rng(407)
    B, Hq, Hkv, L, D = 3, 4, 2, 20, 8
    sl = np.array([20, 7, 1], np.int32)
    q = draw(rng, (B, Hq, L, D), 1.0, "bf16")
    k = draw(rng, (B, Hkv, L, D), 1.0, "bf16")
    v = draw(rng, (B, Hkv, L, D), 1.0, "bf16")
    for causal, W in ((False, 0), (True, 0), (False, 6)):
        clean = oracle.prefill(q, k, v, scale=0.35, causal=causal, seq_lens=sl, window=W)
        kp, vp, qp = k.copy(), v.copy(), q.copy()
        for b in range(B):
            kp[b, :, sl[b]:] = BF16_NAN
            vp[b, :, sl[b]:] = BF16_NAN
            qp[b, :, sl[b]:] = BF16_NAN
        dirty = oracle.prefill(qp, kp, vp, scale=0.35, causal=causal, seq_lens=sl, window=W)
        assert np.array_equal(clean, dirty), "poisoned padding changed the result"
        for b in range(B):
            n = sl[b]
            assert np.all(clean[b, :, n:] == 0.0)
            trunc = oracle.prefill(q[b:b + 1, :, :n], k[b:b + 1, :, :n], v[b:b + 1, :, :n], scale=0.35,
                                   causal=causal, window=W)
            _close(clean[b:b + 1, :, :n], trunc, 0.0, "padded == truncated")


def pin_gqa_equals_repeated_mha(oracle):
    rng = _rng(408)
    B, Hq, Hkv, L, D = 2, 8, 2, 13, 8
    q = draw(rng, (B, Hq, L, D), 1.0, "bf16")
    k = draw(rng, (B, Hkv, L, D), 1.0, "bf16")
    v = draw(rng, (B, Hkv, L, D), 1.0, "bf16")
    g = oracle.prefill(q, k, v, scale=0.3, causal=True, window=5)
    m = oracle.prefill(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), scale=0.3,
                       causal=True, window=5)
    _close(g, m, 0.0, "GQA vs repeated K/V")


def pin_chunked_prefill(oracle):
    """Rows [P, P+n) of a causal prefill == a prefill of those rows at pos_offset P over keys
    [0, P+n)."""
    rng = _rng(409)
    B, Hq, Hkv, L, D = 1, 4, 2, 24, 8
    q = draw(rng, (B, Hq, L, D), 1.0, "f32")
    k = draw(rng, (B, Hkv, L, D), 1.0, "f32")
    v = draw(rng, (B, Hkv, L, D), 1.0, "f32")
    for W in (0, 6):
        full = oracle.prefill(q, k, v, scale=0.4, causal=True, window=W)
        for P, n in ((0, 5), (5, 7), (12, 12), (23, 1)):
            part = oracle.prefill(q[:, :, P:P + n], k[:, :, :P + n], v[:, :, :P + n], scale=0.4, causal=True,
                                  pos_offset=P, window=W)
            _close(part, full[:, :, P:P + n], 0.0, f"chunk P={P} n={n} W={W}")


def pin_permutation_invariance(oracle):
    rng = _rng(410)
    q = draw(rng, (1, 2, 9, 8), 1.0, "f32")
    k = draw(rng, (1, 2, 9, 8), 1.0, "f32")
    v = draw(rng, (1, 2, 9, 8), 1.0, "f32")
    perm = rng.permutation(9)
    a = oracle.prefill(q, k, v, scale=0.5, causal=False)
    b = oracle.prefill(q, k[:, :, perm], v[:, :, perm], scale=0.5, causal=False)
    _close(a, b, 1e-14, "joint K/V permutation")
    # a plain key permutation without moving V must change the result
    c = oracle.prefill(q, k[:, :, perm], v, scale=0.5, causal=False)
    assert np.max(np.abs(a - c)) > 1e-6


def pin_decode_matches_prefill_row(oracle):
    """Decode of item b == the last row of a causal prefill over that item's first
    kv_lens[b] keys; cache slots past kv_len are never read."""
    rng = _rng(411)
    B, Hq, Hkv, cap, L, D = 3, 4, 2, 12, 10, 8
    q = draw(rng, (B, Hq, D), 1.0, "bf16")
    k = draw(rng, (B, Hkv, cap, D), 1.0, "bf16")
    v = draw(rng, (B, Hkv, cap, D), 1.0, "bf16")
    kl = np.array([10, 1, 6], np.int32)
    k[:, :, L:] = BF16_NAN
    v[:, :, L:] = BF16_NAN
    for W in (0, 4):
        out = oracle.decode(q, k, v, kv_len=L, scale=0.3, kv_lens=kl, window=W)
        for b in range(B):
            n = kl[b]
            pre = oracle.prefill(q[b:b + 1, :, None, :], k[b:b + 1, :, :n], v[b:b + 1, :, :n], scale=0.3,
                                 causal=True, pos_offset=n - 1, window=W)
            _close(out[b], pre[0, :, 0], 0.0, f"decode item {b} W={W}")
            one = oracle.decode(q[b:b + 1], k[b:b + 1], v[b:b + 1], kv_len=L, scale=0.3, kv_lens=kl[b:b + 1],
                                window=W)
            _close(out[b], one[0], 0.0, "batched decode == single-item decode")


def pin_rows_entry(oracle):
    """The sampled-rows entry points reproduce the full computations."""
    rng = _rng(412)
    q = draw(rng, (2, 4, 15, 8), 1.0, "bf16")
    k = draw(rng, (2, 2, 15, 8), 1.0, "bf16")
    v = draw(rng, (2, 2, 15, 8), 1.0, "bf16")
    full = oracle.prefill(q, k, v, scale=0.3, causal=True, seq_lens=[15, 8], window=0)
    rows = np.array([[0, 0, 0], [1, 3, 14], [1, 2, 7], [0, 1, 9]], np.int32)
    part = oracle.prefill(q, k, v, scale=0.3, causal=True, seq_lens=[15, 8], rows=rows)
    _close(part, full[rows[:, 0], rows[:, 1], rows[:, 2]], 0.0, "prefill rows")
    qd = draw(rng, (2, 4, 8), 1.0, "bf16")
    fd = oracle.decode(qd, k, v, kv_len=15, scale=0.3, pos_offset=14)
    pd = oracle.decode(qd, k, v, kv_len=15, scale=0.3, pos_offset=14, rows=[[1, 3], [0, 0]])
    _close(pd, fd[[1, 0], [3, 0]], 0.0, "decode rows")


def pin_bf16_widening(oracle):
    """bf16 inputs are read exactly: the bf16 run equals the fp32 run on the widened values."""
    rng = _rng(413)
    x32 = rng.standard_normal((3, 1, 2, 6, 8), dtype=np.float32)
    xb = bf16_bits_from_f32(x32)
    xw = f32_from_bf16_bits(xb)
    a = oracle.prefill(xb[0], xb[1], xb[2], scale=0.5, causal=True)
    b = oracle.prefill(xw[0], xw[1], xw[2], scale=0.5, causal=True)
    _close(a, b, 0.0, "bf16 vs widened fp32")


# ---------------------------------------------------------------------------
# per-item caches and the fused append (ferrum-kernels `Backend`, Provided Methods:
# `kv_cache_append_batched_per_cache`, `flash_attention_batched_per_cache`)

def _per_item_caches(rng, B, Hkv, cap, D, dtype):
    k = [draw(rng, (Hkv, cap, D), 1.0, dtype) for _ in range(B)]
    v = [draw(rng, (Hkv, cap, D), 1.0, dtype) for _ in range(B)]
    return k, v


def pin_append_writes_one_slot(oracle):
    """Only slot cache_lens[b] of every kv head of item b changes, to the new row; items
    without room and the input caches are left as they were (checked slot by slot)."""
    rng = _rng(500)
    B, Hkv, cap, D = 4, 2, 6, 8
    kc, vc = _per_item_caches(rng, B, Hkv, cap, D, "bf16")
    kn = draw(rng, (B, Hkv, D), 1.0, "bf16")
    vn = draw(rng, (B, Hkv, D), 1.0, "bf16")
    keep_k, keep_v = [c.copy() for c in kc], [c.copy() for c in vc]
    lens = np.array([0, 5, 6, -1], np.int32)   # first slot, last slot, full, negative
    ko, vo = oracle.append(kc, vc, kn, vn, lens)
    for b in range(B):
        assert np.array_equal(kc[b], keep_k[b]) and np.array_equal(vc[b], keep_v[b]), "input cache modified"
        for h in range(Hkv):
            for j in range(cap):
                written = j == lens[b] and 0 <= lens[b] < cap
                want_k = kn[b, h] if written else keep_k[b][h, j]
                want_v = vn[b, h] if written else keep_v[b][h, j]
                assert np.array_equal(ko[b][h, j], want_k), f"K item {b} head {h} slot {j}"
                assert np.array_equal(vo[b][h, j], want_v), f"V item {b} head {h} slot {j}"


def pin_decode_append_brute_force(oracle):
    """Append + decode == brute-force attention of the query at position L over the
    explicitly concatenated keys [cache[:L], new] (causal, and the last-W window)."""
    for n, (B, Hq, Hkv, cap, D, lens, W) in enumerate([
            (3, 4, 2, 7, 8, [0, 3, 6], 0),
            (3, 2, 1, 9, 4, [8, 2, 9], 3),
            (2, 6, 3, 5, 8, [4, -2], 2)]):
        rng = _rng(510 + n)
        q = draw(rng, (B, Hq, D), 1.0, "f32")
        kc, vc = _per_item_caches(rng, B, Hkv, cap, D, "f32")
        kn = draw(rng, (B, Hkv, D), 1.0, "f32")
        vn = draw(rng, (B, Hkv, D), 1.0, "f32")
        scale = 0.45 + 0.1 * n
        out, _, _ = oracle.decode_append(q, kn, vn, kc, vc, np.array(lens, np.int32), scale=scale, window=W)
        for b in range(B):
            L = lens[b]
            if not 0 <= L < cap:
                _close(out[b], np.zeros((Hq, D)), 0.0, f"case {n} item {b} without room")
                continue
            kf = np.concatenate([kc[b][:, :L], kn[b][:, None]], axis=1)[None]
            vf = np.concatenate([vc[b][:, :L], vn[b][:, None]], axis=1)[None]
            ref = brute.decode(q[b:b + 1], kf, vf, kv_len=L + 1, scale=scale, pos_offset=L, window=W)
            _close(out[b], np.array(ref[0]), 1e-12, f"case {n} item {b}")


def pin_decode_append_first_token(oracle):
    """An empty cache (length 0): the new token is the only key, so the output is its V
    row for every query head of the group, and a one-key window changes nothing."""
    rng = _rng(520)
    B, Hq, Hkv, cap, D = 2, 4, 2, 3, 8
    q = draw(rng, (B, Hq, D), 1.0, "bf16")
    kc, vc = _per_item_caches(rng, B, Hkv, cap, D, "bf16")
    kn = draw(rng, (B, Hkv, D), 1.0, "bf16")
    vn = draw(rng, (B, Hkv, D), 1.0, "bf16")
    for W in (0, 1):
        out, _, _ = oracle.decode_append(q, kn, vn, kc, vc, np.zeros(B, np.int32), scale=0.3, window=W)
        for b in range(B):
            for h in range(Hq):
                _close(out[b, h], _f64(vn[b, h // 2]), 0.0, f"first token W={W} item {b} head {h}")


def pin_decode_per_cache_equals_single_calls(oracle):
    """One batched call over per-item caches == one single-item call per item on its own
    cache (the loop the batched call replaces), and == brute force."""
    rng = _rng(530)
    B, Hq, Hkv, cap, D = 3, 4, 2, 10, 8
    q = draw(rng, (B, Hq, D), 1.0, "f32")
    kc, vc = _per_item_caches(rng, B, Hkv, cap, D, "f32")
    lens = np.array([10, 1, 7], np.int32)
    for W in (0, 3):
        out = oracle.decode_per_cache(q, kc, vc, lens, scale=0.6, window=W)
        for b in range(B):
            one = oracle.decode(q[b:b + 1], kc[b][None], vc[b][None], kv_len=cap, scale=0.6, pos_offset=lens[b] - 1,
                                window=W)
            _close(out[b], one[0], 0.0, f"per-cache item {b} W={W}")
            ref = brute.decode(q[b:b + 1], kc[b][None], vc[b][None], kv_len=cap, scale=0.6, kv_lens=lens[b:b + 1],
                               window=W)
            _close(out[b], np.array(ref[0]), 1e-12, f"per-cache brute item {b} W={W}")


# ---------------------------------------------------------------------------
# unpadded (varlen) batches (ripvec-core `Driver`, `prepare_batch_unpadded`)

def pin_varlen_brute_force(oracle):
    """Token-major unpadded batch == brute force on each item's own tokens, with the
    item's rows gathered by explicit per-token loops (not by a reshape)."""
    for n, (lens, Hq, Hkv, D, causal, W) in enumerate([
            ([3, 0, 5, 1], 2, 1, 4, True, 0),
            ([6, 2], 4, 2, 8, False, 0),
            ([5, 4, 7], 2, 2, 4, False, 3),
            ([7, 1, 4], 2, 1, 8, True, 3)]):
        rng = _rng(540 + n)
        T = sum(lens)
        q = draw(rng, (T, Hq, D), 1.0, "f32")
        k = draw(rng, (T, Hkv, D), 1.0, "f32")
        v = draw(rng, (T, Hkv, D), 1.0, "f32")
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        got = oracle.prefill_varlen(q, k, v, cu, scale=0.55, causal=causal, window=W)
        for b, L in enumerate(lens):
            if L == 0:
                continue
            t0 = int(cu[b])
            qi = np.zeros((1, Hq, L, D), np.float32)
            ki = np.zeros((1, Hkv, L, D), np.float32)
            vi = np.zeros((1, Hkv, L, D), np.float32)
            for t in range(L):
                for h in range(Hq):
                    qi[0, h, t] = q[t0 + t, h]
                for h in range(Hkv):
                    ki[0, h, t] = k[t0 + t, h]
                    vi[0, h, t] = v[t0 + t, h]
            ref = np.array(brute.attention(qi, ki, vi, scale=0.55, causal=causal, window=W))
            for t in range(L):
                for h in range(Hq):
                    _close(got[t0 + t, h], ref[0, h, t], 1e-12, f"varlen case {n} item {b} token {t} head {h}")


def pin_varlen_item_order(oracle):
    """Reordering the items (moving each item's token block with it) reorders the output
    blocks the same way; a single-token item outputs its own V row."""
    rng = _rng(550)
    lens = [4, 1, 6]
    Hq, Hkv, D = 4, 2, 8
    T = sum(lens)
    q = draw(rng, (T, Hq, D), 1.0, "bf16")
    k = draw(rng, (T, Hkv, D), 1.0, "bf16")
    v = draw(rng, (T, Hkv, D), 1.0, "bf16")
    cu = np.array([0, 4, 5, 11], np.int32)
    a = oracle.prefill_varlen(q, k, v, cu, scale=0.4, causal=True)
    order = [2, 0, 1]
    blocks = [np.arange(cu[b], cu[b + 1]) for b in order]
    idx = np.concatenate(blocks)
    cu2 = np.concatenate([[0], np.cumsum([lens[b] for b in order])]).astype(np.int32)
    b2 = oracle.prefill_varlen(q[idx], k[idx], v[idx], cu2, scale=0.4, causal=True)
    _close(b2, a[idx], 0.0, "item reorder")
    for h in range(Hq):
        _close(a[4, h], _f64(v[4, h // 2]), 0.0, "single-token item")


# ---------------------------------------------------------------------------
# fp16 inputs (ripvec-core `Driver`, the `_f16` twins: half storage)

def pin_f16_every_value_exact(oracle):
    """Every fp16 bit pattern is read exactly: with one key, out = that key's V row, so a
    V row holding all 63488 finite fp16 values must come back as numpy's widening of
    them; the infinities and a NaN come back as themselves."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = bits[(bits & 0x7C00) != 0x7C00]
    special = np.array([0x7C00, 0xFC00, 0x7E00], np.uint16)   # +inf, -inf, NaN
    for vals in (finite, special):
        n = vals.size
        v = vals.view(np.float16).reshape(1, 1, 1, n)
        z = np.zeros((1, 1, 1, n), np.float16)
        out = oracle.prefill(z, z, v, scale=1.0)
        want = vals.view(np.float16).astype(np.float64)
        assert np.array_equal(out[0, 0, 0], want, equal_nan=True), "fp16 decode"


def pin_f16_widening(oracle):
    """fp16 inputs equal their exact fp32 widening (numpy's conversion)."""
    rng = _rng(414)
    x = rng.standard_normal((3, 2, 4, 9, 8), dtype=np.float32).astype(np.float16)
    a = oracle.prefill(x[0], x[1][:, :2], x[2][:, :2], scale=0.5, causal=True, window=5)
    w = x.astype(np.float32)
    b = oracle.prefill(w[0], w[1][:, :2], w[2][:, :2], scale=0.5, causal=True, window=5)
    _close(a, b, 0.0, "fp16 vs widened fp32")


def pin_token_major_brute_force(oracle):
    """Token-major prefill == brute force on head-major copies built element by element."""
    rng = _rng(560)
    B, Lq, Lk, Hq, Hkv, D = 2, 5, 7, 4, 2, 4
    q = draw(rng, (B, Lq, Hq, D), 1.0, "f32")
    k = draw(rng, (B, Lk, Hkv, D), 1.0, "f32")
    v = draw(rng, (B, Lk, Hkv, D), 1.0, "f32")
    got = oracle.prefill_token_major(q, k, v, scale=0.6, causal=True, pos_offset=2, seq_lens=[7, 5], window=4)
    qh = np.zeros((B, Hq, Lq, D), np.float32)
    kh = np.zeros((B, Hkv, Lk, D), np.float32)
    vh = np.zeros((B, Hkv, Lk, D), np.float32)
    for b in range(B):
        for t in range(Lq):
            for h in range(Hq):
                qh[b, h, t] = q[b, t, h]
        for t in range(Lk):
            for h in range(Hkv):
                kh[b, h, t] = k[b, t, h]
                vh[b, h, t] = v[b, t, h]
    ref = np.array(brute.attention(qh, kh, vh, scale=0.6, causal=True, pos_offset=2, seq_lens=[7, 5], window=4))
    for b in range(B):
        for t in range(Lq):
            for h in range(Hq):
                _close(got[b, t, h], ref[b, h, t], 1e-12, f"token-major item {b} token {t} head {h}")


PINS = {name[4:]: fn for name, fn in sorted(globals().items()) if name.startswith("pin_") and callable(fn)}
