"""The pins are strong enough: plant plausible mistakes in the oracle (on the
CPU, by monkeypatching) and check that some pin fails for each."""
import numpy as np
import pytest

import oracle
import oracle.ref as ref
import tests.test_oracle_pins as pins

F64 = np.float64


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(ref, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def deq_wrong_group(q, s, group=128):
    n, k = q.shape
    idx = np.arange(k) % (k // group)                 # k mod G instead of k div 128
    return q.astype(F64) * s.astype(F64)[:, idx]


def rope_interleaved(z, pos, theta=1e6):
    z = np.asarray(z, dtype=F64)
    d = z.shape[-1]
    i = np.arange(d // 2, dtype=F64)
    phi = np.asarray(pos, dtype=F64)[..., None] * theta ** (-2 * i / d)
    phi = phi[..., None, :]
    c, s = np.cos(phi), np.sin(phi)
    ev, od = z[..., 0::2], z[..., 1::2]
    out = np.empty_like(z)
    out[..., 0::2] = ev * c - od * s
    out[..., 1::2] = ev * s + od * c
    return out


def rope_wrong_sign(z, pos, theta=1e6):
    return ref.__dict__["_orig_rope"](z, -np.asarray(pos, dtype=F64), theta)


def rmsnorm_eps_outside(x, w, eps=1e-6):
    x = np.asarray(x, dtype=F64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * np.asarray(w, F64)


def swiglu_swapped(g, u):
    return ref.silu(u) * np.asarray(g, F64)


def _attn_variant(gqa_mod=False, no_scale=False, ignore_table=False):
    orig = ref.__dict__["_orig_paged"]

    def f(q, k_pool, v_pool, page_table, ctx, scale, page=16):
        if no_scale:
            scale = 1.0
        if ignore_table:
            page_table = np.arange(len(page_table))
        if gqa_mod:
            n_qh, n_kvh = q.shape[0], k_pool.shape[1]
            grp = n_qh // n_kvh
            # head h reads kv head h mod n_kvh: reorder heads so orig's h // grp mapping does it
            perm = np.array([(h % n_kvh) * grp + h // n_kvh for h in range(n_qh)])
            out = orig(np.asarray(q)[np.argsort(perm)], k_pool, v_pool, page_table, ctx, scale, page)
            return out[perm]
        return orig(q, k_pool, v_pool, page_table, ctx, scale, page)
    return f


def quantize_int4_absmax_8(w, group=128):
    w = np.asarray(w, dtype=np.float16)
    n, k = w.shape
    wg = w.astype(F64).reshape(n, k // group, group)
    scales = (np.max(np.abs(wg), axis=2) / 8.0).astype(np.float16)     # /8 instead of /7
    s64 = scales.astype(F64)[:, :, None]
    r = np.where(s64 > 0, np.rint(wg / np.where(s64 > 0, s64, 1.0)), 0.0)
    return np.clip(r, -8, 7).astype(np.int8).reshape(n, k), scales


def quantize_int4_round_away(w, group=128):
    w = np.asarray(w, dtype=np.float16)
    n, k = w.shape
    wg = w.astype(F64).reshape(n, k // group, group)
    scales = (np.max(np.abs(wg), axis=2) / 7.0).astype(np.float16)
    s64 = scales.astype(F64)[:, :, None]
    qq = np.where(s64 > 0, wg / np.where(s64 > 0, s64, 1.0), 0.0)
    r = np.sign(qq) * np.floor(np.abs(qq) + 0.5)                          # ties away from zero
    return np.clip(r, -8, 7).astype(np.int8).reshape(n, k), scales


def quantize_act_per_tensor(x, group=128):
    x = np.asarray(x, dtype=np.float16).astype(np.float32)
    sc = np.float32(np.max(np.abs(x)) / np.float32(127.0))                 # one scale for all groups
    codes = np.clip(np.rint(x / sc), -127, 127).astype(np.int8) if sc > 0 else np.zeros(x.shape, np.int8)
    return codes, np.full(x.shape[0] // group, sc, np.float32)


def quantize_act_round_away(x, group=128):
    x = np.asarray(x, dtype=np.float16)
    k = x.shape[0]
    xg = x.astype(np.float32).reshape(k // group, group)
    scales = (np.max(np.abs(xg), axis=1) / np.float32(127.0)).astype(np.float32)
    codes = np.zeros_like(xg, dtype=np.int8)
    for g in range(k // group):
        if scales[g] == 0:
            continue
        qq = (xg[g] / scales[g]).astype(np.float32)
        codes[g] = np.clip(np.sign(qq) * np.floor(np.abs(qq) + 0.5), -127, 127).astype(np.int8)
    return codes.reshape(k), scales


def gemv_w4a8_scale_of_first_group(q, s, xq, xs, group=128):
    xdeq = np.asarray(xq, dtype=F64) * float(xs[0])                        # group scale ignored
    return ref.deq(q, s, group) @ xdeq


MUTANTS = [
    ("deq", deq_wrong_group, [pins.test_deq_group_indexing]),
    ("rope", rope_interleaved, [pins.test_rope_closed_forms]),
    ("rope", rope_wrong_sign, [pins.test_rope_closed_forms]),
    ("rmsnorm", rmsnorm_eps_outside, [pins.test_rmsnorm_closed_forms]),
    ("swiglu", swiglu_swapped, [pins.test_swiglu_closed_forms]),
    ("paged_attention", "gqa_mod", [pins.test_attention_gqa_mapping]),
    ("paged_attention", "no_scale", [pins.test_attention_two_token_closed_form]),
    ("paged_attention", "ignore_table", [pins.test_attention_page_table_shuffle_invariance_and_tail]),
    ("quantize_int4", quantize_int4_absmax_8, [pins.test_quantize_int4_rational_bruteforce,
                                               pins.test_quantize_int4_bounds]),
    ("quantize_int4", quantize_int4_round_away, [pins.test_quantize_int4_rational_bruteforce]),
    ("quantize_act_int8", quantize_act_per_tensor, [pins.test_quantize_act_rational_bruteforce,
                                                   pins.test_quantize_act_bounds_and_extremes]),
    ("quantize_act_int8", quantize_act_round_away, [pins.test_quantize_act_rational_bruteforce]),
    ("gemv_w4a8", gemv_w4a8_scale_of_first_group, [pins.test_gemv_w4a8_rational_and_reduces_to_w4a16]),
]


@pytest.mark.parametrize("i", range(len(MUTANTS)))
def test_planted_mistake_is_caught(monkeypatch, i):
    name, fn, tests = MUTANTS[i]
    monkeypatch.setitem(ref.__dict__, "_orig_rope", ref.rope)
    monkeypatch.setitem(ref.__dict__, "_orig_paged", ref.paged_attention)
    if isinstance(fn, str):
        fn = _attn_variant(**{fn: True})
    _patch(monkeypatch, name, fn)
    for t in tests:
        with pytest.raises(AssertionError):
            t()
