"""Python binding of libmi_attn (MI355X / gfx950 attention).

Argument marshalling only: each function checks the tensors it is given, turns them
into device pointers and sizes, and calls the C entry point of the same name
(declared in include/mi_attn.h) on the current HIP stream.  Every step of the
computation runs in the library's kernels; there is no fallback of any kind, and a
missing library or GPU raises.

    attn_prefill(q, k, v, out=None, *, pos_offset=0, seq_lens=None, window=0,
                 causal=False, scale=None)
    attn_prefill_token_major(q, k, v, out=None, *, pos_offset=0, seq_lens=None, window=0,
                             causal=False, scale=None)
    attn_prefill_varlen(q, k, v, cu_seqlens, max_seqlen=None, out=None, *, window=0,
                        causal=False, scale=None)
    attn_decode(q, k_cache, v_cache, out=None, *, kv_len=None, pos_offset=None,
                kv_lens=None, window=0, scale=None, workspace=None)
    attn_decode_per_cache(q, k_caches, v_caches, kv_lens, out=None, *, window=0,
                          scale=None, workspace=None)
    attn_decode_append(q, k_new, v_new, k_caches, v_caches, cache_lens, out=None, *,
                       window=0, scale=None, workspace=None)
    attn_decode_append_qkv(qkv, k_caches, v_caches, cache_lens, out=None, *, window=0,
                           scale=None, workspace=None)
    attn_decode_noalloc(q, k_cache, v_cache, out=None, *, kv_len=None, pos_offset=None,
                        kv_lens=None, window=0, scale=None)
    attn_decode_workspace_bytes(batch, q_heads, kv_heads, kv_len, head_dim)
    attn_last_error(), attn_version()

Layouts: q [batch, q_heads, q_len, head_dim]; k, v [batch, kv_heads, kv_len, head_dim]
(token-major: q, out [batch, q_len, q_heads, head_dim], k, v [batch, kv_len, kv_heads,
head_dim]; unpadded: q, out [tokens, q_heads, head_dim], k, v [tokens, kv_heads, head_dim]);
decode caches [batch, kv_heads, capacity, head_dim] (head-major); the per-cache calls
take one [kv_heads, capacity, head_dim] cache per item.  scale defaults to
1/sqrt(head_dim).
"""
from __future__ import annotations

import ctypes
import math
from pathlib import Path

LIBRARY = Path(__file__).resolve().parent / "libmi_attn.so"

MI_ATTN_F32, MI_ATTN_BF16, MI_ATTN_F16 = 0, 1, 2
MI_ATTN_OK, MI_ATTN_ERR_INVALID, MI_ATTN_ERR_UNSUPPORTED, MI_ATTN_ERR_HIP = 0, 1, 2, 3

EXPORTS = ("attn_prefill", "attn_prefill_token_major", "attn_prefill_varlen", "attn_decode", "attn_decode_noalloc",
           "attn_decode_per_cache", "attn_decode_append", "attn_decode_append_qkv", "attn_decode_workspace_bytes",
           "attn_last_error", "attn_version")


class MiAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """Load libmi_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIBRARY.exists():
            raise RuntimeError(f"{LIBRARY} is not built; run `python -m head_attention_02_amd.build`")
        lib = ctypes.CDLL(str(LIBRARY))
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.attn_prefill.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp, i, i, f, i, vp]
        lib.attn_prefill.restype = i
        lib.attn_prefill_token_major.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp, i, i, f, i, vp]
        lib.attn_prefill_token_major.restype = i
        lib.attn_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
        lib.attn_prefill_varlen.restype = i
        lib.attn_decode.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp, i, f, i, vp, sz, vp]
        lib.attn_decode.restype = i
        lib.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp, i, f, i, vp]
        lib.attn_decode_noalloc.restype = i
        lib.attn_decode_per_cache.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, i, f, i, vp, sz, vp]
        lib.attn_decode_per_cache.restype = i
        lib.attn_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, i, f, i, vp, sz, vp]
        lib.attn_decode_append.restype = i
        lib.attn_decode_append_qkv.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, i, f, i, vp, sz, vp]
        lib.attn_decode_append_qkv.restype = i
        lib.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.attn_decode_workspace_bytes.restype = sz
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_version.argtypes = []
        lib.attn_version.restype = i
        _lib = lib
    return _lib


def attn_version() -> int:
    return library().attn_version()


def attn_last_error() -> str:
    return library().attn_last_error().decode()


def attn_decode_workspace_bytes(batch: int, q_heads: int, kv_heads: int, kv_len: int, head_dim: int) -> int:
    return int(library().attn_decode_workspace_bytes(batch, q_heads, kv_heads, kv_len, head_dim))


def _check(status: int) -> None:
    if status != MI_ATTN_OK:
        raise MiAttnError(status, attn_last_error())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MI_ATTN_BF16
    if t.dtype == torch.float32:
        return MI_ATTN_F32
    if t.dtype == torch.float16:
        return MI_ATTN_F16
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16, float16 or float32)")


def _dev(t, name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def attn_prefill(q, k, v, out=None, *, pos_offset: int = 0, seq_lens=None, window: int = 0,
                 causal: bool = False, scale: float | None = None, stream=None):
    """Prefill attention; returns `out` [batch, q_heads, q_len, head_dim]."""
    return _prefill_padded(False, q, k, v, out, pos_offset, seq_lens, window, causal, scale, stream)


def attn_prefill_token_major(q, k, v, out=None, *, pos_offset: int = 0, seq_lens=None, window: int = 0,
                             causal: bool = False, scale: float | None = None, stream=None):
    """Prefill attention on token-major tensors: q [batch, q_len, q_heads, head_dim], k, v
    [batch, kv_len, kv_heads, head_dim]; returns `out` [batch, q_len, q_heads, head_dim]."""
    return _prefill_padded(True, q, k, v, out, pos_offset, seq_lens, window, causal, scale, stream)


def _prefill_padded(token_major, q, k, v, out, pos_offset, seq_lens, window, causal, scale, stream):
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q and k, v must be 4-D of one layout, k and v of one shape")
    if token_major:
        B, Lq, Hq, D = q.shape
        Bk, Lk, Hkv, Dk = k.shape
    else:
        B, Hq, Lq, D = q.shape
        Bk, Hkv, Lk, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree on batch or head_dim")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or seq_lens.numel() != B):
        raise ValueError("seq_lens must be an int32 tensor of batch elements")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    fn = library().attn_prefill_token_major if token_major else library().attn_prefill
    st = fn(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), B, Hq, Hkv, Lq, Lk, D, pos_offset,
            _dev(seq_lens, "seq_lens"), window, int(bool(causal)), float(scale), dt, _stream(stream))
    _check(st)
    return out


def attn_prefill_varlen(q, k, v, cu_seqlens, max_seqlen: int | None = None, out=None, *, window: int = 0,
                        causal: bool = False, scale: float | None = None, stream=None):
    """Prefill on an unpadded, token-major batch; returns `out` [tokens, q_heads, head_dim].
    Without `max_seqlen` it is read from cu_seqlens on the host (one device sync)."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [tokens,Hq,D] and k, v [tokens,Hkv,D]")
    T, Hq, D = q.shape
    Tk, Hkv, Dk = k.shape
    if Tk != T or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree on tokens or head_dim")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of batch + 1 offsets")
    B = cu_seqlens.numel() - 1
    if max_seqlen is None:
        c = cu_seqlens.cpu()
        max_seqlen = int((c[1:] - c[:-1]).max()) if B > 0 else 0
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = library().attn_prefill_varlen(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                                       _dev(cu_seqlens, "cu_seqlens"), B, int(max_seqlen), Hq, Hkv, D, window,
                                       int(bool(causal)), float(scale), dt, _stream(stream))
    _check(st)
    return out


def _decode_args(q, k_cache, v_cache, out, kv_len, pos_offset, kv_lens):
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,Hq,D] and the caches [B,Hkv,capacity,D]")
    B, Hq, D = q.shape
    Bk, Hkv, cap, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError("q and the caches disagree on batch or head_dim")
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    if kv_len is None:
        kv_len = cap
    if pos_offset is None:
        pos_offset = kv_len - 1
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if kv_lens is not None and (kv_lens.dtype != torch.int32 or kv_lens.numel() != B):
        raise ValueError("kv_lens must be an int32 tensor of batch elements")
    return B, Hq, Hkv, cap, D, dt, kv_len, pos_offset, out


def attn_decode(q, k_cache, v_cache, out=None, *, kv_len: int | None = None, pos_offset: int | None = None,
                kv_lens=None, window: int = 0, scale: float | None = None, workspace=None, stream=None):
    """Decode attention of one token per (item, head); returns `out` [batch, q_heads, head_dim]."""
    torch = _torch()
    B, Hq, Hkv, cap, D, dt, kv_len, pos_offset, out = _decode_args(q, k_cache, v_cache, out, kv_len, pos_offset,
                                                                   kv_lens)
    need = attn_decode_workspace_bytes(B, Hq, Hkv, kv_len, D) if Hq % Hkv == 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = library().attn_decode(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(out, "out"),
                               B, Hq, Hkv, kv_len, cap, D, pos_offset, _dev(kv_lens, "kv_lens"), window,
                               float(scale), dt, _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    _check(st)
    return out


def attn_decode_noalloc(q, k_cache, v_cache, out=None, *, kv_len: int | None = None, pos_offset: int | None = None,
                        kv_lens=None, window: int = 0, scale: float | None = None, stream=None):
    """attn_decode with the split partial states in the library's per-GPU scratch: the
    library allocates nothing.  Pass `out` as well to keep the whole call free of
    allocations (else it is allocated here, by torch, as for the other calls)."""
    B, Hq, Hkv, cap, D, dt, kv_len, pos_offset, out = _decode_args(q, k_cache, v_cache, out, kv_len, pos_offset,
                                                                   kv_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = library().attn_decode_noalloc(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                       _dev(out, "out"), B, Hq, Hkv, kv_len, cap, D, pos_offset,
                                       _dev(kv_lens, "kv_lens"), window, float(scale), dt, _stream(stream))
    _check(st)
    return out


class CacheTable:
    """The device array of per-item cache pointers the per-cache calls take, built once.

    Passing one of these instead of a list of tensors saves the host-to-device copy of
    the pointer array on every call (a decode loop builds it once per set of caches).
    It keeps the cache tensors alive."""

    def __init__(self, caches, batch: int | None = None, name: str = "caches"):
        if isinstance(caches, (list, tuple)):
            first = caches[0]
            B = len(caches)
        else:
            first, B = caches, caches.shape[0]
        if batch is not None and B != batch:
            raise ValueError(f"{name}: {B} caches for batch {batch}")
        self.ptrs, self.dims = _cache_pointers(caches, B, name, first.dtype, first.device)
        self.batch, self.dtype, self.caches = B, first.dtype, caches


def _cache_pointers(caches, B: int, name: str, dtype, device):
    """Device int64 tensor of `B` cache base pointers, and (kv_heads, capacity, head_dim).

    `caches` is a list of `B` contiguous tensors [kv_heads, capacity, head_dim] (one per
    item, any allocation), one contiguous [B, kv_heads, capacity, head_dim] tensor (its
    items' bases are used), or a CacheTable."""
    torch = _torch()
    if isinstance(caches, CacheTable):
        if caches.batch != B or caches.dtype != dtype:
            raise ValueError(f"{name}: cache table of batch {caches.batch}, {caches.dtype} for batch {B}, {dtype}")
        return caches.ptrs, caches.dims
    if isinstance(caches, (list, tuple)):
        if len(caches) != B:
            raise ValueError(f"{name}: {len(caches)} caches for batch {B}")
        shapes = {tuple(c.shape) for c in caches}
        if len(shapes) != 1 or len(next(iter(shapes))) != 3:
            raise ValueError(f"{name}: every cache must be [kv_heads, capacity, head_dim] of one shape")
        for c in caches:
            _dev(c, name, dtype)
            if c.data_ptr() % 16:
                raise ValueError(f"{name}: caches must be 16-byte aligned")
        ptrs = [c.data_ptr() for c in caches]
        dims = next(iter(shapes))
    else:
        if caches.dim() != 4 or caches.shape[0] != B:
            raise ValueError(f"{name}: expected [B, kv_heads, capacity, head_dim] or a list of caches")
        _dev(caches, name, dtype)
        step = caches.stride(0) * caches.element_size()
        ptrs = [caches.data_ptr() + b * step for b in range(B)]
        dims = tuple(caches.shape[1:])
    return torch.tensor(ptrs, dtype=torch.int64, device=device), dims


def _keep_for(stream, *tensors) -> None:
    """Keeps the per-call pointer arrays alive until the call's kernels have read them.

    They are freed when the call returns.  On torch's current stream (stream None) the
    allocator orders their reuse after the kernels already; on any other stream -- a torch
    stream object or a raw hipStream_t handle -- each array is recorded on that stream,
    so the allocator does not hand its memory out before the stream's queued work ran."""
    if stream is None:
        return
    torch = _torch()
    s = stream if hasattr(stream, "cuda_stream") else torch.cuda.ExternalStream(int(stream))
    for t in tensors:
        t.record_stream(s)


def _decode_common(q, k_caches, v_caches, lens, out, workspace, what: str):
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be [B,Hq,D]")
    B, Hq, D = q.shape
    kp, kd = _cache_pointers(k_caches, B, "k_caches", q.dtype, q.device)
    vp, vd = _cache_pointers(v_caches, B, "v_caches", q.dtype, q.device)
    if kd != vd:
        raise ValueError("K and V caches differ in shape")
    Hkv, cap, Dk = kd
    if Dk != D:
        raise ValueError("q and the caches disagree on head_dim")
    if lens is None or lens.dtype != torch.int32 or lens.numel() != B:
        raise ValueError(f"{what} must be an int32 tensor of batch elements")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    need = attn_decode_workspace_bytes(B, Hq, Hkv, cap, D) if Hq % Hkv == 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return B, Hq, Hkv, cap, D, kp, vp, out, workspace, ws_bytes


def attn_decode_per_cache(q, k_caches, v_caches, kv_lens, out=None, *, window: int = 0,
                          scale: float | None = None, workspace=None, stream=None):
    """Decode over one cache per item (a list of [kv_heads, capacity, head_dim] tensors);
    returns `out` [batch, q_heads, head_dim]."""
    dt = _dtype_code(q)
    B, Hq, Hkv, cap, D, kp, vp, out, workspace, ws_bytes = _decode_common(q, k_caches, v_caches, kv_lens, out,
                                                                          workspace, "kv_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = library().attn_decode_per_cache(_dev(q, "q"), _dev(kp, "k_caches"), _dev(vp, "v_caches"), _dev(out, "out"),
                                         B, Hq, Hkv, cap, D, _dev(kv_lens, "kv_lens"), window, float(scale), dt,
                                         _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    _keep_for(stream, kp, vp)
    _check(st)
    return out


def attn_decode_append(q, k_new, v_new, k_caches, v_caches, cache_lens, out=None, *, window: int = 0,
                       scale: float | None = None, workspace=None, stream=None):
    """Append the new token's K/V rows [batch, kv_heads, head_dim] at slot cache_lens[b] of
    each item's caches, then decode its query over them; returns `out`.  The caches are
    modified in place; cache_lens is not (the caller advances it)."""
    dt = _dtype_code(q)
    B, Hq, Hkv, cap, D, kp, vp, out, workspace, ws_bytes = _decode_common(q, k_caches, v_caches, cache_lens, out,
                                                                          workspace, "cache_lens")
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        if tuple(t.shape) != (B, Hkv, D) or t.dtype != q.dtype:
            raise ValueError(f"{nm} must be [batch, kv_heads, head_dim] of q's dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = library().attn_decode_append(_dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                      _dev(kp, "k_caches"), _dev(vp, "v_caches"), _dev(out, "out"), B, Hq, Hkv,
                                      cap, D, _dev(cache_lens, "cache_lens"), window, float(scale), dt,
                                      _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    _keep_for(stream, kp, vp)
    _check(st)
    return out


def attn_decode_append_qkv(qkv, k_caches, v_caches, cache_lens, out=None, *, window: int = 0,
                           scale: float | None = None, workspace=None, stream=None):
    """attn_decode_append with the new token's query, key and value read from one fused row
    per item: qkv [batch, q_heads + 2 * kv_heads, head_dim], contiguous (the query heads,
    then the key heads, then the value heads); returns `out` [batch, q_heads, head_dim]."""
    dt = _dtype_code(qkv)
    if qkv.dim() != 3 or not qkv.is_contiguous():
        raise ValueError("qkv must be a contiguous [batch, q_heads + 2 * kv_heads, head_dim] tensor")
    _, (Hkv, _, _) = _cache_pointers(k_caches, qkv.shape[0], "k_caches", qkv.dtype, qkv.device)
    Hq = qkv.shape[1] - 2 * Hkv
    if Hq < 1:
        raise ValueError("qkv holds no query head beside the 2 * kv_heads key and value rows")
    if out is None:
        out = _torch().empty((qkv.shape[0], Hq, qkv.shape[2]), dtype=qkv.dtype, device=qkv.device)
    B, Hq, Hkv, cap, D, kp, vp, out, workspace, ws_bytes = _decode_common(qkv[:, :Hq], k_caches, v_caches,
                                                                          cache_lens, out, workspace, "cache_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = library().attn_decode_append_qkv(_dev(qkv, "qkv"), _dev(kp, "k_caches"), _dev(vp, "v_caches"),
                                          _dev(out, "out"), B, Hq, Hkv, cap, D, _dev(cache_lens, "cache_lens"),
                                          window, float(scale), dt, _dev(workspace, "workspace"), ws_bytes,
                                          _stream(stream))
    _keep_for(stream, kp, vp)
    _check(st)
    return out
