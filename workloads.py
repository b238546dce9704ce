"""Seeded synthetic inputs for attention, shared by the tests and the benchmark.

This module draws random numbers and stores them; it holds none of the attention
arithmetic.  Both the GPU path and the oracle receive the arrays it makes.

Recipe (every workload): ``rng = numpy.random.default_rng(seed)`` (PCG64); draw the
per-item lengths first when the workload has them, then Q, K and V in that order, each
``rng.standard_normal(shape, dtype=float32) * sigma``.  bf16 tensors are the fp32
draws rounded to the nearest bf16, ties to even, and are stored as their raw uint16
bits.  Padded positions keep their random values.

The five named workloads are the shapes the pages' backends run attention on: a tiny
fp32 causal check, a BERT-base encoder batch with padding, a ModernBERT-style local
(banded) layer, a causal GQA prefill and a batched GQA decode over a head-major cache.
Two more are the BERT batch in the unpadded token-major layout and that decode with the
new token's K/V row appended to the cache first.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to fp32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)


def draw(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    """One tensor of i.i.d. N(0, sigma^2) values: float32, float16, or bf16 bits (uint16)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    if dtype == "f16":
        return x.astype(np.float16)   # numpy rounds to nearest, ties to even
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill", "prefill_token_major", "prefill_varlen", "decode" or "decode_append"
    batch: int
    q_heads: int
    kv_heads: int
    q_len: int                # 1 for decode
    kv_len: int
    head_dim: int
    dtype: str                # "f32", "bf16" or "f16"
    sigma: float
    causal: bool
    window: int = 0
    pos_offset: int = 0
    capacity: int = 0         # decode: cache slots per (item, kv head); 0 = kv_len
    seq_len_range: tuple | None = None  # (lo, hi) inclusive: per-item lengths drawn first
    scale: float = field(default=0.0)
    seed: int = 0

    @property
    def attn_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.head_dim)


WORKLOADS = {
    "tiny_causal_f32": Workload("tiny_causal_f32", "prefill", 1, 2, 2, 64, 64, 32, "f32", 1.0, True,
                                scale=1.0 / math.sqrt(32), seed=1),
    "bert_base_padded": Workload("bert_base_padded", "prefill", 32, 12, 12, 512, 512, 64, "bf16", 1.0,
                                 False, seq_len_range=(16, 512), seed=2),
    "banded_w128_s8192": Workload("banded_w128_s8192", "prefill", 8, 12, 12, 8192, 8192, 64, "bf16", 1.0,
                                  False, window=128, seed=3),
    "causal_gqa_s4096": Workload("causal_gqa_s4096", "prefill", 1, 32, 8, 4096, 4096, 128, "bf16", 0.5,
                                 True, scale=1.0 / math.sqrt(128), seed=4),
    "gqa_decode_kv8192": Workload("gqa_decode_kv8192", "decode", 64, 32, 8, 1, 8192, 128, "bf16", 1.0,
                                  True, pos_offset=8191, capacity=8192, seed=5),
    # the causal GQA prefill and the GQA decode with fp16 inputs (the pages' _f16 twins)
    "causal_gqa_s4096_f16": Workload("causal_gqa_s4096_f16", "prefill", 1, 32, 8, 4096, 4096, 128, "f16", 0.5,
                                     True, scale=1.0 / math.sqrt(128), seed=4),
    "gqa_decode_kv8192_f16": Workload("gqa_decode_kv8192_f16", "decode", 64, 32, 8, 1, 8192, 128, "f16", 1.0,
                                      True, pos_offset=8191, capacity=8192, seed=5),
    # the causal GQA prefill on token-major tensors q/out [B, L, Hq, D], k/v [B, L, Hkv, D]
    "causal_gqa_s4096_token_major": Workload("causal_gqa_s4096_token_major", "prefill_token_major", 1, 32, 8, 4096,
                                             4096, 128, "bf16", 0.5, True, scale=1.0 / math.sqrt(128), seed=4),
    # the BERT-shaped batch without padding: the same item lengths, tokens concatenated
    # token-major ([tokens, heads, head_dim]) with cu_seqlens boundaries
    "bert_base_varlen": Workload("bert_base_varlen", "prefill_varlen", 32, 12, 12, 512, 512, 64, "bf16", 1.0,
                                 False, seq_len_range=(16, 512), seed=2),
    # the same decode step with the new token's K/V row appended to each item's cache
    # first: 8191 tokens already cached, the new one goes to slot 8191
    "gqa_decode_append_kv8192": Workload("gqa_decode_append_kv8192", "decode_append", 64, 32, 8, 1, 8192, 128,
                                         "bf16", 1.0, True, pos_offset=8191, capacity=8192, seed=6),
}


def item_lengths(w: Workload):
    """The per-item lengths a workload draws first (the same values make_inputs returns),
    without drawing the tensors; None when the workload has none."""
    if w.seq_len_range is None:
        return None
    lo, hi = w.seq_len_range
    return np.random.default_rng(w.seed).integers(lo, hi, endpoint=True, size=w.batch).astype(np.int32)


def make_inputs(w: Workload) -> dict:
    """Arrays for a workload, in the draw order of the recipe above.

    prefill: q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D], seq_lens [B] int32 or None
    prefill_token_major: q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D], seq_lens as for prefill
    prefill_varlen: q [T,Hq,D], k/v [T,Hkv,D] token-major over the items' T tokens (drawn
             after the lengths), seq_lens [B], cu_seqlens [B+1] int32
    decode:  q [B,Hq,D], k/v caches [B,Hkv,capacity,D], kv_lens None
    decode_append: as decode, then the new rows k_new/v_new [B,Hkv,D] (drawn after the
             caches) and cache_lens [B] int32 (the per-item lengths when drawn, else
             pos_offset for every item)
    """
    rng = np.random.default_rng(w.seed)
    seq_lens = None
    if w.seq_len_range is not None:
        lo, hi = w.seq_len_range
        seq_lens = rng.integers(lo, hi, endpoint=True, size=w.batch).astype(np.int32)
    if w.kind == "prefill_varlen":
        lens = seq_lens if seq_lens is not None else np.full(w.batch, w.q_len, np.int32)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = int(cu[-1])
        q = draw(rng, (T, w.q_heads, w.head_dim), w.sigma, w.dtype)
        k = draw(rng, (T, w.kv_heads, w.head_dim), w.sigma, w.dtype)
        v = draw(rng, (T, w.kv_heads, w.head_dim), w.sigma, w.dtype)
        return {"q": q, "k": k, "v": v, "seq_lens": lens, "cu_seqlens": cu}
    if w.kind == "prefill_token_major":
        q = draw(rng, (w.batch, w.q_len, w.q_heads, w.head_dim), w.sigma, w.dtype)
        k = draw(rng, (w.batch, w.kv_len, w.kv_heads, w.head_dim), w.sigma, w.dtype)
        v = draw(rng, (w.batch, w.kv_len, w.kv_heads, w.head_dim), w.sigma, w.dtype)
        return {"q": q, "k": k, "v": v, "seq_lens": seq_lens}
    if w.kind == "prefill":
        q = draw(rng, (w.batch, w.q_heads, w.q_len, w.head_dim), w.sigma, w.dtype)
        k = draw(rng, (w.batch, w.kv_heads, w.kv_len, w.head_dim), w.sigma, w.dtype)
        v = draw(rng, (w.batch, w.kv_heads, w.kv_len, w.head_dim), w.sigma, w.dtype)
        return {"q": q, "k": k, "v": v, "seq_lens": seq_lens}
    cap = w.capacity or w.kv_len
    q = draw(rng, (w.batch, w.q_heads, w.head_dim), w.sigma, w.dtype)
    k = draw(rng, (w.batch, w.kv_heads, cap, w.head_dim), w.sigma, w.dtype)
    v = draw(rng, (w.batch, w.kv_heads, cap, w.head_dim), w.sigma, w.dtype)
    if w.kind == "decode_append":
        k_new = draw(rng, (w.batch, w.kv_heads, w.head_dim), w.sigma, w.dtype)
        v_new = draw(rng, (w.batch, w.kv_heads, w.head_dim), w.sigma, w.dtype)
        cache_lens = seq_lens if seq_lens is not None else np.full(w.batch, w.pos_offset, np.int32)
        return {"q": q, "k": k, "v": v, "k_new": k_new, "v_new": v_new, "cache_lens": cache_lens}
    return {"q": q, "k": k, "v": v, "kv_lens": seq_lens}


def random_prefill(seed: int, batch: int, q_heads: int, kv_heads: int, q_len: int, kv_len: int,
                   head_dim: int, dtype: str = "bf16", sigma: float = 1.0, seq_len_range=None) -> dict:
    """Ad-hoc prefill inputs with the same recipe (used by parity and edge-case tests)."""
    w = Workload("adhoc", "prefill", batch, q_heads, kv_heads, q_len, kv_len, head_dim, dtype, sigma,
                 False, seq_len_range=seq_len_range, seed=seed)
    return make_inputs(w)


def random_decode(seed: int, batch: int, q_heads: int, kv_heads: int, capacity: int, head_dim: int,
                  dtype: str = "bf16", sigma: float = 1.0, kv_len_range=None) -> dict:
    """Ad-hoc decode inputs with the same recipe; kv_len_range draws per-item lengths."""
    w = Workload("adhoc", "decode", batch, q_heads, kv_heads, 1, capacity, head_dim, dtype, sigma, True,
                 capacity=capacity, seq_len_range=kv_len_range, seed=seed)
    return make_inputs(w)
