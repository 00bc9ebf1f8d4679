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


MUTANTS = [
    ("deq", deq_wrong_group, [pins.test_deq_group_indexing]),
    ("rope", rope_interleaved, [pins.test_rope_closed_forms]),
    ("rope", rope_wrong_sign, [pins.test_rope_closed_forms]),
    ("rmsnorm", rmsnorm_eps_outside, [pins.test_rmsnorm_closed_forms]),
    ("swiglu", swiglu_swapped, [pins.test_swiglu_closed_forms]),
    ("paged_attention", "gqa_mod", [pins.test_attention_gqa_mapping]),
    ("paged_attention", "no_scale", [pins.test_attention_two_token_closed_form]),
    ("paged_attention", "ignore_table", [pins.test_attention_page_table_shuffle_invariance_and_tail]),
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
