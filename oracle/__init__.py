"""Python handle on the fp64 CPU attention oracle (``attn_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The oracle is the reference the GPU library is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with ``head_attention_02_amd``
and the GPU library never calls it.

Arrays are numpy.  A float32 array is read as fp32, a float16 array as fp16; a uint16
array is read as the raw bits of bf16 values.  Every result is float64 and unrounded.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "attn_oracle.c"
LIBRARY = HERE / "liboracle_attn.so"

_F32, _BF16, _F16 = 0, 1, 2
_dbl_p = ctypes.POINTER(ctypes.c_double)
_i32_p = ctypes.POINTER(ctypes.c_int32)


def compile_library(source: Path = SOURCE, output: Path = LIBRARY) -> Path:
    """Compile the oracle with gcc into a shared library (plain C, -O2, pthreads)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-o", str(output), str(source), "-lm"]
    subprocess.run(cmd, check=True)
    return output


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    vp, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.oracle_prefill.argtypes = [vp, vp, vp, _dbl_p, i, i, i, i, i, i, i, i, _i32_p, i, i, d, i]
    lib.oracle_prefill.restype = i
    lib.oracle_prefill_rows.argtypes = [vp, vp, vp, _dbl_p, i, i, i, i, i, i, i, i, _i32_p, i, i, d,
                                        _i32_p, ctypes.c_int64, i]
    lib.oracle_prefill_rows.restype = i
    lib.oracle_decode.argtypes = [vp, vp, vp, _dbl_p, i, i, i, i, i, i, i, i, _i32_p, i, d, _i32_p,
                                  ctypes.c_int64, i]
    lib.oracle_decode.restype = i
    lib.oracle_prefill_probs.argtypes = [vp, vp, vp, _dbl_p, _dbl_p, i, i, i, i, i, i, i, i, _i32_p,
                                         i, i, d, i, i, i]
    lib.oracle_prefill_probs.restype = ctypes.c_int64
    return lib


def _dtype_code(*arrays: np.ndarray) -> int:
    kinds = {a.dtype for a in arrays}
    if kinds == {np.dtype(np.float32)}:
        return _F32
    if kinds == {np.dtype(np.uint16)}:
        return _BF16
    if kinds == {np.dtype(np.float16)}:
        return _F16
    raise TypeError(f"oracle inputs must all be float32, all float16 or all bf16 bits (uint16), got {kinds}")


def _ptr(a: np.ndarray | None, ctype=ctypes.c_void_p):
    if a is None:
        return None
    if ctype is ctypes.c_void_p:
        return a.ctypes.data_as(ctypes.c_void_p)
    return a.ctypes.data_as(ctype)


def _default_threads() -> int:
    return len(os.sched_getaffinity(0))


class Oracle:
    """The oracle library behind a numpy interface.  ``path`` selects another build
    of the same source (the mutation tests load deliberately broken copies)."""

    def __init__(self, path: Path | str | None = None):
        if path is None:
            path = LIBRARY
            if not Path(path).exists():
                compile_library()
        self.path = Path(path)
        self.lib = _bind(ctypes.CDLL(str(self.path)))
        self.threads_used = 0

    # ---- prefill ---------------------------------------------------------------
    def prefill(self, q, k, v, *, scale: float, causal: bool = False, pos_offset: int = 0,
                seq_lens=None, window: int = 0, rows=None, nthreads: int | None = None) -> np.ndarray:
        """q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] -> [B,Hq,Lq,D] float64, or [n,D] for ``rows``
        given as an (n, 3) array of (b, h, i)."""
        q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
        dt = _dtype_code(q, k, v)
        B, Hq, Lq, D = q.shape
        Bk, Hkv, Lk, Dk = k.shape
        if (Bk, Dk) != (B, D) or v.shape != k.shape:
            raise ValueError("shape mismatch between q, k and v")
        sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
        nt = nthreads or _default_threads()
        if rows is None:
            out = np.zeros((B, Hq, Lq, D), np.float64)
            ret = self.lib.oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out, _dbl_p), dt, B, Hq, Hkv,
                                          Lq, Lk, D, pos_offset, _ptr(sl, _i32_p), window, int(causal),
                                          float(scale), nt)
        else:
            r = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
            out = np.zeros((r.shape[0], D), np.float64)
            ret = self.lib.oracle_prefill_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(out, _dbl_p), dt, B, Hq,
                                               Hkv, Lq, Lk, D, pos_offset, _ptr(sl, _i32_p), window,
                                               int(causal), float(scale), _ptr(r, _i32_p), r.shape[0], nt)
        if ret < 0:
            raise ValueError(f"oracle_prefill rejected its arguments (code {ret})")
        self.threads_used = ret
        return out

    def prefill_token_major(self, q, k, v, *, scale: float, causal: bool = False, pos_offset: int = 0,
                            seq_lens=None, window: int = 0, nthreads: int | None = None) -> np.ndarray:
        """The prefill definition on token-major tensors: q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D]
        -> [B,Lq,Hq,D] float64 (the layout before ferrum-kernels Backend's head-major
        conversion and after its `transpose_head_to_token`)."""
        qh = np.ascontiguousarray(np.asarray(q).transpose(0, 2, 1, 3))
        kh = np.ascontiguousarray(np.asarray(k).transpose(0, 2, 1, 3))
        vh = np.ascontiguousarray(np.asarray(v).transpose(0, 2, 1, 3))
        out = self.prefill(qh, kh, vh, scale=scale, causal=causal, pos_offset=pos_offset, seq_lens=seq_lens,
                           window=window, nthreads=nthreads)
        return np.ascontiguousarray(out.transpose(0, 2, 1, 3))

    def prefill_varlen(self, q, k, v, cu_seqlens, *, scale: float, causal: bool = False, window: int = 0,
                       nthreads: int | None = None) -> np.ndarray:
        """Unpadded batch (ripvec-core `Driver`, `prepare_batch_unpadded`): tokens of all
        items concatenated, token-major q [T,Hq,D], k/v [T,Hkv,D]; item b is tokens
        [cu_seqlens[b], cu_seqlens[b+1]) and attends over its own tokens only, query i at
        position i.  Returns [T,Hq,D] float64; rows of no item stay 0."""
        q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
        T, Hq, D = q.shape
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        out = np.zeros((T, Hq, D), np.float64)
        for b in range(len(cu) - 1):
            t0, t1 = int(cu[b]), int(cu[b + 1])
            if t1 <= t0:
                continue
            # this item alone in the head-major layout [1, heads, len, D]
            qi = np.ascontiguousarray(q[t0:t1].transpose(1, 0, 2))[None]
            ki = np.ascontiguousarray(k[t0:t1].transpose(1, 0, 2))[None]
            vi = np.ascontiguousarray(v[t0:t1].transpose(1, 0, 2))[None]
            oi = self.prefill(qi, ki, vi, scale=scale, causal=causal, window=window, nthreads=nthreads)
            out[t0:t1] = oi[0].transpose(1, 0, 2)
        return out

    # ---- decode ----------------------------------------------------------------
    def decode(self, q, k_cache, v_cache, *, kv_len: int, scale: float, pos_offset: int = 0,
               kv_lens=None, window: int = 0, rows=None, nthreads: int | None = None) -> np.ndarray:
        """q [B,Hq,D], caches [B,Hkv,capacity,D] -> [B,Hq,D] float64 (or [n,D] for
        ``rows`` given as (b, h) pairs)."""
        q, k_cache, v_cache = (np.ascontiguousarray(x) for x in (q, k_cache, v_cache))
        dt = _dtype_code(q, k_cache, v_cache)
        B, Hq, D = q.shape
        Bk, Hkv, cap, Dk = k_cache.shape
        if (Bk, Dk) != (B, D) or v_cache.shape != k_cache.shape:
            raise ValueError("shape mismatch between q and the caches")
        kl = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int32)
        nt = nthreads or _default_threads()
        if rows is None:
            out = np.zeros((B, Hq, D), np.float64)
            rp, n = None, 0
        else:
            r2 = np.asarray(rows, dtype=np.int32).reshape(-1, 2)
            r = np.ascontiguousarray(np.concatenate([r2, np.zeros((r2.shape[0], 1), np.int32)], axis=1))
            out = np.zeros((r.shape[0], D), np.float64)
            rp, n = _ptr(r, _i32_p), r.shape[0]
        ret = self.lib.oracle_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out, _dbl_p), dt, B, Hq,
                                     Hkv, kv_len, cap, D, pos_offset, _ptr(kl, _i32_p), window,
                                     float(scale), rp, n, nt)
        if ret < 0:
            raise ValueError(f"oracle_decode rejected its arguments (code {ret})")
        self.threads_used = ret
        return out

    # ---- per-item caches and the cache append ------------------------------------
    # ferrum-kernels `Backend` page, Provided Methods: `kv_cache_append_batched_per_cache`
    # writes item i's new head-major row [nkv, hd] into its own cache [nkv, capacity, hd]
    # at the offset cache_lens[i]; `flash_attention_batched_per_cache` attends M items'
    # queries over their own caches with per-item lengths, replacing M single-item calls.

    @staticmethod
    def append(k_caches, v_caches, k_new, v_new, cache_lens):
        """Caches after appending one token per item: lists of `B` arrays
        [Hkv, capacity, D] (copies; the inputs are not modified).  Row cache_lens[b] of
        every kv head of item b becomes k_new[b] / v_new[b].  An item whose offset lies
        outside [0, capacity) has no room and keeps its caches unchanged."""
        ko = [np.array(c, copy=True) for c in k_caches]
        vo = [np.array(c, copy=True) for c in v_caches]
        for b, n in enumerate(np.asarray(cache_lens, dtype=np.int64)):
            cap = ko[b].shape[1]
            if 0 <= n < cap:
                ko[b][:, n, :] = k_new[b]
                vo[b][:, n, :] = v_new[b]
        return ko, vo

    def decode_per_cache(self, q, k_caches, v_caches, kv_lens, *, scale: float, window: int = 0,
                         rows=None, nthreads: int | None = None) -> np.ndarray:
        """q [B,Hq,D]; k_caches / v_caches: `B` arrays [Hkv, capacity, D], one per item;
        item b has kv_lens[b] keys and its query at kv_lens[b] - 1.  This is the batched
        decode over the items' caches side by side."""
        K = np.stack([np.asarray(c) for c in k_caches])
        V = np.stack([np.asarray(c) for c in v_caches])
        return self.decode(q, K, V, kv_len=K.shape[2], scale=scale, kv_lens=kv_lens, window=window, rows=rows,
                           nthreads=nthreads)

    def decode_append(self, q, k_new, v_new, k_caches, v_caches, cache_lens, *, scale: float, window: int = 0,
                      rows=None, nthreads: int | None = None):
        """The two steps in order: append each item's new K/V row at cache_lens[b], then
        attend its query (at position cache_lens[b]) over the cache holding it.  Returns
        (out, k_caches, v_caches).  Items without room have no keys: output 0."""
        ko, vo = self.append(k_caches, v_caches, k_new, v_new, cache_lens)
        cap = ko[0].shape[1] if ko else 0
        cl = np.asarray(cache_lens, dtype=np.int64)
        lens = np.where((cl >= 0) & (cl < cap), cl + 1, 0).astype(np.int32)
        out = self.decode_per_cache(q, ko, vo, lens, scale=scale, window=window, rows=rows, nthreads=nthreads)
        return out, ko, vo

    # ---- inspection --------------------------------------------------------------
    def prefill_probs(self, q, k, v, b: int, h: int, i: int, *, scale: float, causal: bool = False,
                      pos_offset: int = 0, seq_lens=None, window: int = 0):
        """Softmax weights [Lk] of one row, its output [D] and its key-set size."""
        q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
        dt = _dtype_code(q, k, v)
        B, Hq, Lq, D = q.shape
        _, Hkv, Lk, _ = k.shape
        sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
        probs = np.zeros(max(Lk, 1), np.float64)
        out = np.zeros(D, np.float64)
        n = self.lib.oracle_prefill_probs(_ptr(q), _ptr(k), _ptr(v), _ptr(probs, _dbl_p), _ptr(out, _dbl_p),
                                          dt, B, Hq, Hkv, Lq, Lk, D, pos_offset, _ptr(sl, _i32_p), window,
                                          int(causal), float(scale), b, h, i)
        if n < 0:
            raise ValueError(f"oracle_prefill_probs rejected its arguments (code {n})")
        return probs[:Lk], out, int(n)


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``attn_oracle.c`` in this directory (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
