"""libmi_attn on the CPU: it loads, exports every declared symbol, and its host-side
validation rejects bad arguments before touching the GPU (no kernel is launched here)."""
import ctypes
import math
import re
from pathlib import Path

import pytest

import head_attention_02_amd as mi

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "mi_attn.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(mi.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    lib = mi.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    version = int(re.search(r"#define MI_ATTN_VERSION (\d+)", HEADER.read_text()).group(1))
    assert mi.attn_version() == version


def test_workspace_query():
    # few (item, kv head) units: the key range is split, one fp32 partial state
    # (head_dim + 2 values) per (item, query head, split)
    n = mi.attn_decode_workspace_bytes(2, 32, 8, 8192, 128)
    per_split = 2 * 32 * (128 + 2) * 4
    assert n > per_split and n % per_split == 0
    # enough units to fill the GPU without splitting: no workspace at all
    assert mi.attn_decode_workspace_bytes(64, 32, 8, 8192, 128) == 0
    assert mi.attn_decode_workspace_bytes(0, 32, 8, 8192, 128) == 0
    assert mi.attn_decode_workspace_bytes(64, 30, 8, 8192, 128) == 0
    assert mi.attn_decode_workspace_bytes(64, 32, 8, 8192, 96) == 0


FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: validation fails first


def prefill(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, batch=2, q_heads=8, kv_heads=2, q_len=16, kv_len=16,
                head_dim=64, pos_offset=0, seq_lens=None, window=0, causal=1, scale=0.125, dtype=mi.MI_ATTN_BF16,
                stream=None)
    args.update(kw)
    return mi.library().attn_prefill(*args.values())


def decode(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, batch=2, q_heads=8, kv_heads=2, kv_len=16, capacity=16,
                head_dim=64, pos_offset=15, kv_lens=None, window=0, scale=0.125, dtype=mi.MI_ATTN_BF16,
                ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return mi.library().attn_decode(*args.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q_heads=6, kv_heads=4), mi.MI_ATTN_ERR_INVALID, "not a multiple"),
    (dict(kv_heads=0), mi.MI_ATTN_ERR_INVALID, "must be >= 1"),
    (dict(pos_offset=4), mi.MI_ATTN_ERR_INVALID, "exceeds kv_len"),
    (dict(pos_offset=-1), mi.MI_ATTN_ERR_INVALID, "exceeds kv_len"),
    (dict(q_len=-1), mi.MI_ATTN_ERR_INVALID, "negative size"),
    (dict(window=-3), mi.MI_ATTN_ERR_INVALID, "negative"),
    (dict(scale=math.inf), mi.MI_ATTN_ERR_INVALID, "not finite"),
    (dict(head_dim=96), mi.MI_ATTN_ERR_UNSUPPORTED, "head_dim 96"),
    (dict(dtype=7), mi.MI_ATTN_ERR_UNSUPPORTED, "dtype"),
    (dict(q=None), mi.MI_ATTN_ERR_INVALID, "null"),
    (dict(out=ctypes.c_void_p(0x100004)), mi.MI_ATTN_ERR_INVALID, "aligned"),
])
def test_prefill_validation(kw, status, msg):
    assert prefill(**kw) == status
    err = mi.attn_last_error()
    assert err.startswith("attn_prefill: ") and msg in err


def test_prefill_empty_calls_are_ok_without_a_gpu():
    assert prefill(batch=0) == mi.MI_ATTN_OK
    assert prefill(q_len=0, q=None) == mi.MI_ATTN_OK


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q_heads=6, kv_heads=4), mi.MI_ATTN_ERR_INVALID, "not a multiple"),
    (dict(kv_len=17), mi.MI_ATTN_ERR_INVALID, "capacity"),
    (dict(kv_len=0), mi.MI_ATTN_ERR_INVALID, "capacity"),
    (dict(pos_offset=16), mi.MI_ATTN_ERR_INVALID, "pos_offset"),
    (dict(window=-1), mi.MI_ATTN_ERR_INVALID, "negative"),
    (dict(head_dim=48), mi.MI_ATTN_ERR_UNSUPPORTED, "head_dim 48"),
    # 4096 keys of 4 (item, kv head) units are split, so a workspace is needed
    (dict(kv_len=4096, capacity=4096, ws_bytes=16), mi.MI_ATTN_ERR_INVALID, "workspace"),
    (dict(kv_len=4096, capacity=4096, ws=None), mi.MI_ATTN_ERR_INVALID, "workspace"),
    (dict(v=None), mi.MI_ATTN_ERR_INVALID, "null"),
])
def test_decode_validation(kw, status, msg):
    assert decode(**kw) == status
    err = mi.attn_last_error()
    assert err.startswith("attn_decode: ") and msg in err


def test_decode_empty_batch_is_ok_without_a_gpu():
    assert decode(batch=0) == mi.MI_ATTN_OK


def decode_noalloc(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, batch=2, q_heads=8, kv_heads=2, kv_len=16, capacity=16,
                head_dim=64, pos_offset=15, kv_lens=None, window=0, scale=0.125, dtype=mi.MI_ATTN_BF16, stream=None)
    args.update(kw)
    return mi.library().attn_decode_noalloc(*args.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q_heads=6, kv_heads=4), mi.MI_ATTN_ERR_INVALID, "not a multiple"),
    (dict(kv_len=17), mi.MI_ATTN_ERR_INVALID, "capacity"),
    (dict(pos_offset=16), mi.MI_ATTN_ERR_INVALID, "pos_offset"),
    (dict(head_dim=48), mi.MI_ATTN_ERR_UNSUPPORTED, "head_dim 48"),
    (dict(v=None), mi.MI_ATTN_ERR_INVALID, "null"),
    # 511 (item, kv head) units of 8 query heads, split in two: 511 * 8 * 2 * 130 * 4 bytes of
    # partial states, more than the scratch holds
    (dict(batch=511, q_heads=8, kv_heads=1, head_dim=128, kv_len=4096, capacity=4096, pos_offset=4095),
     mi.MI_ATTN_ERR_UNSUPPORTED, "scratch"),
])
def test_decode_noalloc_validation(kw, status, msg):
    """The no-allocation decode validates like attn_decode, and refuses sizes whose
    partial states exceed its fixed scratch -- all before any GPU call."""
    assert decode_noalloc(**kw) == status
    err = mi.attn_last_error()
    assert err.startswith("attn_decode_noalloc: ") and msg in err


def test_decode_noalloc_scratch_limit_matches_the_header():
    limit = int(re.search(r"#define MI_ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", HEADER.read_text())
                .expand(r"\1")) << int(re.search(r"MI_ATTN_NOALLOC_SCRATCH_BYTES \(\d+u << (\d+)\)",
                                                 HEADER.read_text()).group(1))
    assert mi.attn_decode_workspace_bytes(511, 8, 1, 4096, 128) > limit
    # the workload-sized decode needs no scratch at all, a small-batch one fits
    assert mi.attn_decode_workspace_bytes(64, 32, 8, 8192, 128) == 0
    assert 0 < mi.attn_decode_workspace_bytes(2, 16, 4, 3000, 128) <= limit


def test_decode_noalloc_empty_batch_is_ok_without_a_gpu():
    assert decode_noalloc(batch=0) == mi.MI_ATTN_OK


def test_error_message_is_cleared_by_a_good_call():
    assert prefill(kv_heads=3) != mi.MI_ATTN_OK
    assert mi.attn_last_error()
    assert prefill(batch=0) == mi.MI_ATTN_OK
    assert mi.attn_last_error() == ""


def per_cache(**kw):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, out=FAKE, batch=2, q_heads=8, kv_heads=2, capacity=16, head_dim=64,
                kv_lens=FAKE, window=0, scale=0.125, dtype=mi.MI_ATTN_BF16, ws=FAKE, ws_bytes=1 << 30,
                stream=None)
    args.update(kw)
    return mi.library().attn_decode_per_cache(*args.values())


def append(**kw):
    args = dict(q=FAKE, k_new=FAKE, v_new=FAKE, kc=FAKE, vc=FAKE, out=FAKE, batch=2, q_heads=8, kv_heads=2,
                capacity=16, head_dim=64, cache_lens=FAKE, window=0, scale=0.125, dtype=mi.MI_ATTN_BF16, ws=FAKE,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return mi.library().attn_decode_append(*args.values())


COMMON_PER_ITEM_ERRORS = [
    (dict(q_heads=6, kv_heads=4), mi.MI_ATTN_ERR_INVALID, "not a multiple"),
    (dict(capacity=0), mi.MI_ATTN_ERR_INVALID, "capacity"),
    (dict(window=-1), mi.MI_ATTN_ERR_INVALID, "negative"),
    (dict(scale=math.nan), mi.MI_ATTN_ERR_INVALID, "not finite"),
    (dict(head_dim=80), mi.MI_ATTN_ERR_UNSUPPORTED, "head_dim 80"),
    (dict(dtype=5), mi.MI_ATTN_ERR_UNSUPPORTED, "dtype"),
    (dict(kc=None), mi.MI_ATTN_ERR_INVALID, "null"),
    (dict(out=ctypes.c_void_p(0x100008)), mi.MI_ATTN_ERR_INVALID, "aligned"),
    (dict(vc=ctypes.c_void_p(0x100004)), mi.MI_ATTN_ERR_INVALID, "aligned"),
    # 4096 slots of 4 (item, kv head) units are split, so a workspace is needed
    (dict(capacity=4096, ws_bytes=16), mi.MI_ATTN_ERR_INVALID, "workspace"),
]


@pytest.mark.parametrize("kw,status,msg", COMMON_PER_ITEM_ERRORS + [
    (dict(kv_lens=None), mi.MI_ATTN_ERR_INVALID, "null"),
])
def test_decode_per_cache_validation(kw, status, msg):
    assert per_cache(**kw) == status
    err = mi.attn_last_error()
    assert err.startswith("attn_decode_per_cache: ") and msg in err


@pytest.mark.parametrize("kw,status,msg", COMMON_PER_ITEM_ERRORS + [
    (dict(cache_lens=None), mi.MI_ATTN_ERR_INVALID, "null"),
    (dict(k_new=None), mi.MI_ATTN_ERR_INVALID, "new K/V"),
    (dict(v_new=ctypes.c_void_p(0x100002)), mi.MI_ATTN_ERR_INVALID, "new K/V"),
])
def test_decode_append_validation(kw, status, msg):
    assert append(**kw) == status
    err = mi.attn_last_error()
    assert err.startswith("attn_decode_append: ") and msg in err


def append_qkv(**kw):
    args = dict(qkv=FAKE, kc=FAKE, vc=FAKE, out=FAKE, batch=2, q_heads=8, kv_heads=2, capacity=16, head_dim=64,
                cache_lens=FAKE, window=0, scale=0.125, dtype=mi.MI_ATTN_BF16, ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return mi.library().attn_decode_append_qkv(*args.values())


@pytest.mark.parametrize("kw,status,msg", [e for e in COMMON_PER_ITEM_ERRORS if "q_heads" not in e[0]] + [
    (dict(cache_lens=None), mi.MI_ATTN_ERR_INVALID, "null"),
    (dict(qkv=None), mi.MI_ATTN_ERR_INVALID, "null fused row"),
    (dict(qkv=ctypes.c_void_p(0x100004)), mi.MI_ATTN_ERR_INVALID, "aligned"),
    (dict(q_heads=0), mi.MI_ATTN_ERR_INVALID, "head counts"),
    (dict(q_heads=6, kv_heads=4), mi.MI_ATTN_ERR_INVALID, "not a multiple"),
])
def test_decode_append_qkv_validation(kw, status, msg):
    assert append_qkv(**kw) == status
    err = mi.attn_last_error()
    assert err.startswith("attn_decode_append_qkv: ") and msg in err


def test_per_item_empty_batch_is_ok_without_a_gpu():
    assert per_cache(batch=0, kv_lens=None) == mi.MI_ATTN_OK
    assert append(batch=0, k_new=None, v_new=None) == mi.MI_ATTN_OK
    assert append_qkv(batch=0, qkv=None) == mi.MI_ATTN_OK


def varlen(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, cu=FAKE, batch=3, max_seqlen=100, q_heads=8, kv_heads=2,
                head_dim=64, window=0, causal=0, scale=0.125, dtype=mi.MI_ATTN_BF16, stream=None)
    args.update(kw)
    return mi.library().attn_prefill_varlen(*args.values())


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q_heads=6, kv_heads=4), mi.MI_ATTN_ERR_INVALID, "not a multiple"),
    (dict(max_seqlen=-1), mi.MI_ATTN_ERR_INVALID, "negative size"),
    (dict(batch=-2), mi.MI_ATTN_ERR_INVALID, "negative size"),
    (dict(window=-1), mi.MI_ATTN_ERR_INVALID, "negative"),
    (dict(scale=-math.inf), mi.MI_ATTN_ERR_INVALID, "not finite"),
    (dict(head_dim=256), mi.MI_ATTN_ERR_UNSUPPORTED, "head_dim 256"),
    (dict(dtype=3), mi.MI_ATTN_ERR_UNSUPPORTED, "dtype"),
    (dict(cu=None), mi.MI_ATTN_ERR_INVALID, "null"),
    (dict(k=ctypes.c_void_p(0x100002)), mi.MI_ATTN_ERR_INVALID, "aligned"),
    (dict(cu=ctypes.c_void_p(0x100002)), mi.MI_ATTN_ERR_INVALID, "aligned"),
])
def test_prefill_varlen_validation(kw, status, msg):
    assert varlen(**kw) == status
    err = mi.attn_last_error()
    assert err.startswith("attn_prefill_varlen: ") and msg in err


def test_prefill_varlen_empty_calls_are_ok_without_a_gpu():
    assert varlen(batch=0, cu=None) == mi.MI_ATTN_OK
    assert varlen(max_seqlen=0, q=None) == mi.MI_ATTN_OK


def test_token_major_prefill_validation():
    lib = mi.library()
    args = [FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 16, 16, 64, 0, None, 0, 1, 0.125, mi.MI_ATTN_BF16, None]
    bad = list(args)
    bad[5] = 6   # q_heads not a multiple of kv_heads... 6 % 2 == 0, so use kv_heads 4
    bad[6] = 4
    assert lib.attn_prefill_token_major(*bad) == mi.MI_ATTN_ERR_INVALID
    assert mi.attn_last_error().startswith("attn_prefill_token_major: ") and "not a multiple" in mi.attn_last_error()
    bad = list(args)
    bad[10] = 9   # pos_offset + q_len > kv_len
    assert lib.attn_prefill_token_major(*bad) == mi.MI_ATTN_ERR_INVALID
    assert "exceeds kv_len" in mi.attn_last_error()
    empty = list(args)
    empty[4] = 0
    assert lib.attn_prefill_token_major(*empty) == mi.MI_ATTN_OK


def test_binding_fails_loudly_without_the_library(tmp_path):
    """The binding has no fallback: with the library absent, loading it raises."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("mi_copy", mi.__file__)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    m.LIBRARY = tmp_path / "libmi_attn.so"
    m._lib = None
    with pytest.raises(RuntimeError, match="not built"):
        m.library()
    with pytest.raises(RuntimeError, match="not built"):
        m.attn_version()


def test_binding_sources_hold_no_attention_arithmetic():
    """The binding marshals arguments only: no softmax, exp or matmul of its own, and it
    never imports the oracle."""
    src = Path(mi.__file__).read_text()
    for word in ("softmax", "exp(", "matmul", "@", "einsum", "import oracle", "scaled_dot_product"):
        assert word not in src, word


def test_pointer_arrays_are_kept_for_every_stream_kind(monkeypatch):
    """The per-cache calls' device pointer arrays are freed when the call returns; on a
    stream other than torch's current one they must be recorded on that stream -- also
    when the stream comes as a raw hipStream_t integer (wrapped as an external stream)."""
    import torch

    import head_attention_02_amd as mi

    class Arr:
        def __init__(self):
            self.recorded = []

        def record_stream(self, s):
            self.recorded.append(s)

    class TorchStream:
        cuda_stream = 1234

    made = []

    def external(handle):
        made.append(handle)
        return ("external", handle)

    monkeypatch.setattr(torch.cuda, "ExternalStream", external)
    a, b = Arr(), Arr()
    mi._keep_for(None, a, b)              # torch's current stream: ordered by the allocator
    assert a.recorded == [] and b.recorded == []
    ts = TorchStream()
    mi._keep_for(ts, a, b)                # a torch stream object
    assert a.recorded == [ts] and b.recorded == [ts]
    mi._keep_for(0xBEEF, a, b)            # a raw integer handle
    assert made == [0xBEEF]
    assert a.recorded[-1] == ("external", 0xBEEF) and b.recorded[-1] == ("external", 0xBEEF)
