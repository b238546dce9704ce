"""Brute-force attention in pure-Python loops, for pinning the oracle on tiny inputs.

Written independently of the oracle and in a different form: it builds the whole key
set of a row as a Python set from the pages' mask definitions, exponentiates raw
scores without a running maximum, and normalises at the end.  Only for shapes of a
few rows and keys (inputs are small N(0,1) draws, so exp() cannot overflow).

Mask definitions, one per source:
  * causal: row i sees keys 0..i (realizar `cached/attention.rs`,
    `batched_causal_softmax`), shifted by the query's absolute position
    pos_offset + i (ferrum-kernels `Backend`, `qk_norm_rope`);
  * padding: keys at or after the item's valid length are masked (ripvec-core
    `Driver`, `build_attn_mask`); a query row at or past it is padding, output 0
    (ripvec-core `Driver`, `unpad_from_batch`);
  * bidirectional window w: keys with |query_pos - key_pos| > w/2 are masked
    (ripvec-core `Driver`, `fused_scale_mask_softmax_windowed`);
  * causal window w: only the last w valid positions (ferrum-kernels `Backend`,
    `flash_attention_batched_per_cache`).
"""
from __future__ import annotations

import math

import numpy as np

from workloads import f32_from_bf16_bits


def _as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        a = f32_from_bf16_bits(a)
    return np.asarray(a, dtype=np.float64)


def key_set(p: int, valid: int, causal: bool, window: int) -> set:
    if p >= valid:
        return set()
    keys = set(range(valid))
    if causal:
        keys &= set(range(0, p + 1))
    if window:
        if causal:
            keys &= set(range(p - window + 1, p + 1))
        else:
            keys = {j for j in keys if abs(p - j) * 2 <= window - (window % 2)}
    return keys


def attention(q, k, v, *, scale, causal=False, pos_offset=0, seq_lens=None, window=0):
    """q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] (float32 or bf16 bits) -> nested lists [B][Hq][Lq][D]."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    per_kv = Hq // Hkv
    out = []
    for b in range(B):
        valid = Lk if seq_lens is None else min(max(int(seq_lens[b]), 0), Lk)
        ob = []
        for h in range(Hq):
            kh = h // per_kv
            oh = []
            for i in range(Lq):
                keys = sorted(key_set(pos_offset + i, valid, causal, window))
                weights = {}
                for j in keys:
                    s = 0.0
                    for d in range(D):
                        s += float(q[b, h, i, d]) * float(k[b, kh, j, d])
                    weights[j] = math.exp(scale * s)
                z = sum(weights.values())
                row = []
                for d in range(D):
                    acc = 0.0
                    for j in keys:
                        acc += weights[j] * float(v[b, kh, j, d])
                    row.append(acc / z if z > 0 else 0.0)
                oh.append(row)
            ob.append(oh)
        out.append(ob)
    return out


def decode(q, k_cache, v_cache, *, kv_len, scale, pos_offset=0, kv_lens=None, window=0):
    """q [B,Hq,D], caches [B,Hkv,cap,D] -> nested lists [B][Hq][D].  The query of item b
    sits at kv_lens[b]-1 (or pos_offset) and sees the causal prefix of the cache."""
    qa = _as_f64(q)
    B, Hq, D = qa.shape
    res = []
    for b in range(B):
        if kv_lens is None:
            valid, p = kv_len, pos_offset
        else:
            valid = min(max(int(kv_lens[b]), 0), kv_len)
            p = valid - 1
        kb = _as_f64(k_cache[b:b + 1, :, :kv_len])
        vb = _as_f64(v_cache[b:b + 1, :, :kv_len])
        qb = qa[b:b + 1, :, None, :]
        if p < 0:
            res.append([[0.0] * D for _ in range(Hq)])
            continue
        o = attention(qb, kb, vb, scale=scale, causal=True, pos_offset=p, seq_lens=[valid], window=window)
        res.append([o[0][h][0] for h in range(Hq)])
    return res
