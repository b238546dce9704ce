"""attn_decode_noalloc (partial states in the library's per-GPU scratch) against attn_decode
(partial states in a caller workspace): the same kernels and launch plan, so the outputs
must be bit-identical.  Two calls in a row, the second smaller than the first, so the
second runs over the scratch the first left behind; then a call that needs no split."""
import math
import sys

import numpy as np
import pytest

import workloads as W
from gpu_util import to_gpu

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mi():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import head_attention_02_amd as m
    m.library()
    return m


# B, Hq, Hkv, capacity, kv_len, D, lengths, window, dtype
CALLS = [
    (2, 16, 4, 3000, 3000, 128, [3000, 1234], 0, "bf16"),     # 8 units: 12 splits
    (1, 8, 2, 1000, 900, 64, None, 33, "bf16"),                 # smaller, split, windowed
    (3, 8, 8, 520, 520, 32, [520, 7, 0], 0, "f16"),
    (64, 32, 8, 256, 256, 128, None, 0, "bf16"),                # 512 units: no split, no scratch used
]


def _pair(mi, case, seed):
    import torch
    B, Hq, Hkv, cap, L, D, lens, Wn, dt = case
    say(f"no-alloc decode case {case}")
    x = W.random_decode(seed, B, Hq, Hkv, cap, D, dt)
    q, k, v = to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"])
    kl = None if lens is None else to_gpu(np.array(lens, np.int32))
    scale = 1.0 / math.sqrt(D)
    kw = dict(kv_len=L, pos_offset=L - 1, kv_lens=kl, window=Wn, scale=scale)
    need = mi.attn_decode_workspace_bytes(B, Hq, Hkv, L, D)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    want = mi.attn_decode(q, k, v, workspace=ws, **kw)
    out = torch.full_like(q, float("nan"))
    got = mi.attn_decode_noalloc(q, k, v, out, **kw)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"noalloc differs from attn_decode: {case}"
    return need


def test_noalloc_matches_decode_two_calls_second_smaller(mi):
    needs = [_pair(mi, c, 40 + i) for i, c in enumerate(CALLS[:2])]
    assert needs[0] > needs[1] > 0


def test_noalloc_matches_decode_more_shapes(mi):
    for i, c in enumerate(CALLS[2:]):
        _pair(mi, c, 60 + i)
    # and once more the first shape, after the others have used the scratch
    _pair(mi, CALLS[0], 40)
