"""Plant plausible mistakes in copies of the oracle and check that the pins catch each.

Every mutant is a one-place textual change to ``oracle/attn_oracle.c`` (a dropped term,
a wrong sign, index or bound, a transposed or swapped operand), compiled on the CPU
into a temporary library.  The real oracle is never modified.  A mutant that no pin
rejects would mean the pins leave that part of the oracle unchecked.
"""
import numpy as np
import pytest

import oracle
from pins import PINS

MUTANTS = {
    "drop_scale": ("scores[j] = P->scale * dot;", "scores[j] = dot;"),
    "causal_excludes_diagonal": ("if (causal && j > p) return 0;", "if (causal && j >= p) return 0;"),
    "bidir_band_too_narrow": ("if (d > half) return 0;", "if (d >= half) return 0;"),
    "causal_band_too_wide": ("if (p - j >= P->window) return 0;", "if (p - j > P->window) return 0;"),
    "kv_head_interleaved": ("const int kh = h / group;", "const int kh = h % P->kv_heads;"),
    "k_transposed": ("load_elem(P->k, P->dtype, k_row + d)",
                     "load_elem(P->k, P->dtype, kv_head_base * D + (int64_t)d * P->kv_stride + j)"),
    "no_normalisation": ("const double pj = scores[j] / z;", "const double pj = scores[j];"),
    "exp_sign_flipped": ("scores[j] = exp(scores[j] - m);", "scores[j] = exp(m - scores[j]);"),
    "padding_not_masked": ("*nvalid = len;\n    *pos = (int64_t)P->pos_offset + i;",
                           "*nvalid = P->kv_len;\n    *pos = (int64_t)P->pos_offset + i;"),
    "pos_offset_dropped": ("*pos = (int64_t)P->pos_offset + i;", "*pos = (int64_t)i;"),
    "padded_rows_attend": ("if (p >= nvalid) return 0; /* padded query row */", ""),
    "decode_query_one_late": ("*pos = len - 1;", "*pos = len;"),
    "decode_not_causal": ("int causal = P->decode ? 1 : P->causal;", "int causal = P->decode ? 0 : P->causal;"),
    "v_read_from_k": ("load_elem(P->v, P->dtype, v_row + d)", "load_elem(P->k, P->dtype, v_row + d)"),
    "q_head_uses_kv_index": ("(((int64_t)b * P->q_heads + h) * P->q_len + i) * D",
                             "(((int64_t)b * P->q_heads + kh) * P->q_len + i) * D"),
    "last_dim_dropped": ("for (int d = 0; d < D; ++d)\n            dot +=",
                         "for (int d = 0; d < D - 1; ++d)\n            dot +="),
    "f16_exponent_bias": ("ldexp(1024.0 + frac, expo - 25)", "ldexp(1024.0 + frac, expo - 24)"),
    "f16_subnormal_scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -23)"),
    "f16_sign_dropped": ("return sign ? -mag : mag;", "return mag;"),
    "bf16_low_half": ("uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;",
                      "uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 15;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.SOURCE.read_text()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.compile_library(mutant_src, tmp_path / "libmutant.so")
    m = oracle.Oracle(lib)
    caught = []
    for pin_name, pin in PINS.items():
        try:
            pin(m)
        except (AssertionError, ValueError):
            caught.append(pin_name)
    assert caught, f"no pin rejects the mutant {name}"


# ---- the append and per-cache steps (numpy, in oracle/__init__.py) -----------------
# Mutants of these are subclasses that override one step with a plausible mistake.

class _AppendOneLate(oracle.Oracle):
    @staticmethod
    def append(k_caches, v_caches, k_new, v_new, cache_lens):
        return oracle.Oracle.append(k_caches, v_caches, k_new, v_new, np.asarray(cache_lens) + 1)


class _AppendKVSwapped(oracle.Oracle):
    @staticmethod
    def append(k_caches, v_caches, k_new, v_new, cache_lens):
        return oracle.Oracle.append(k_caches, v_caches, v_new, k_new, cache_lens)


class _AppendModifiesInput(oracle.Oracle):
    @staticmethod
    def append(k_caches, v_caches, k_new, v_new, cache_lens):
        for b, n in enumerate(cache_lens):
            if 0 <= n < k_caches[b].shape[1]:
                k_caches[b][:, n, :] = k_new[b]
                v_caches[b][:, n, :] = v_new[b]
        return list(k_caches), list(v_caches)


class _NewKeyNotAttended(oracle.Oracle):
    def decode_append(self, q, k_new, v_new, k_caches, v_caches, cache_lens, *, scale, window=0, rows=None,
                      nthreads=None):
        ko, vo = self.append(k_caches, v_caches, k_new, v_new, cache_lens)
        out = self.decode_per_cache(q, ko, vo, np.maximum(np.asarray(cache_lens, np.int32), 0), scale=scale,
                                    window=window)
        return out, ko, vo


class _NoRoomAttendsAll(oracle.Oracle):
    def decode_append(self, q, k_new, v_new, k_caches, v_caches, cache_lens, *, scale, window=0, rows=None,
                      nthreads=None):
        ko, vo = self.append(k_caches, v_caches, k_new, v_new, cache_lens)
        cap = ko[0].shape[1]
        cl = np.asarray(cache_lens, np.int64)
        lens = np.where(cl < cap, cl + 1, cap).astype(np.int32)
        return self.decode_per_cache(q, ko, vo, lens, scale=scale, window=window), ko, vo


class _PerCacheItemsRotated(oracle.Oracle):
    def decode_per_cache(self, q, k_caches, v_caches, kv_lens, *, scale, window=0, rows=None, nthreads=None):
        k = list(k_caches[1:]) + list(k_caches[:1])
        v = list(v_caches[1:]) + list(v_caches[:1])
        return oracle.Oracle.decode_per_cache(self, q, k, v, kv_lens, scale=scale, window=window)


class _VarlenItemOneLonger(oracle.Oracle):
    def prefill_varlen(self, q, k, v, cu_seqlens, *, scale, causal=False, window=0, nthreads=None):
        cu = np.array(cu_seqlens, np.int64)
        cu[1:-1] += 1
        return oracle.Oracle.prefill_varlen(self, q, k, v, cu, scale=scale, causal=causal, window=window)


class _VarlenHeadsAsTokens(oracle.Oracle):
    def prefill_varlen(self, q, k, v, cu_seqlens, *, scale, causal=False, window=0, nthreads=None):
        T, Hq, D = q.shape
        out = np.zeros((T, Hq, D))
        cu = np.asarray(cu_seqlens, np.int64)
        for b in range(len(cu) - 1):
            t0, t1 = int(cu[b]), int(cu[b + 1])
            if t1 <= t0:
                continue
            L = t1 - t0
            qi = np.ascontiguousarray(q[t0:t1]).reshape(1, Hq, L, D)     # reshape, no transpose
            ki = np.ascontiguousarray(k[t0:t1]).reshape(1, k.shape[1], L, D)
            vi = np.ascontiguousarray(v[t0:t1]).reshape(1, v.shape[1], L, D)
            oi = self.prefill(qi, ki, vi, scale=scale, causal=causal, window=window)
            out[t0:t1] = oi[0].reshape(L, Hq, D)
        return out


class _TokenMajorNoTranspose(oracle.Oracle):
    def prefill_token_major(self, q, k, v, *, scale, causal=False, pos_offset=0, seq_lens=None, window=0,
                            nthreads=None):
        B, Lq, Hq, D = q.shape
        _, Lk, Hkv, _ = k.shape
        out = self.prefill(np.ascontiguousarray(q).reshape(B, Hq, Lq, D), np.ascontiguousarray(k).reshape(B, Hkv, Lk, D),
                           np.ascontiguousarray(v).reshape(B, Hkv, Lk, D), scale=scale, causal=causal,
                           pos_offset=pos_offset, seq_lens=seq_lens, window=window)
        return out.reshape(B, Lq, Hq, D)


PY_MUTANTS = {c.__name__[1:]: c for c in (_TokenMajorNoTranspose, _AppendOneLate, _AppendKVSwapped, _AppendModifiesInput,
                                          _NewKeyNotAttended, _NoRoomAttendsAll, _PerCacheItemsRotated,
                                          _VarlenItemOneLonger, _VarlenHeadsAsTokens)}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_step_mutant_is_caught(name):
    m = PY_MUTANTS[name]()
    caught = []
    for pin_name, pin in PINS.items():
        try:
            pin(m)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin_name)
    assert caught, f"no pin rejects the mutant {name}"
