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


# --------------------------------------------------------------------------
# decoder-block wiring: each mistake is planted in both the sequential layer
# (layer_step, run by decode_step) and the batched teacher-forced pass, and the
# closed-form pins of tests/test_oracle_layer_pins.py must catch it.
# --------------------------------------------------------------------------

import tests.test_oracle_layer_pins as lpins  # noqa: E402

WIRING = ["ln_swap", "bias_after_rope", "mlp_reads_a", "split_qvk", "no_attn_residual",
          "no_mlp_residual", "attn_before_append"]


def _split(dims, y, mut):
    qd, kd = dims.q_dim, dims.kv_dim
    lead = y.shape[:-1]
    q = y[..., :qd]
    if mut == "split_qvk":
        v, k = y[..., qd:qd + kd], y[..., qd + kd:]
    else:
        k, v = y[..., qd:qd + kd], y[..., qd + kd:]
    return (q.reshape(*lead, dims.n_q_heads, dims.head_dim), k.reshape(*lead, dims.n_kv_heads, dims.head_dim),
            v.reshape(*lead, dims.n_kv_heads, dims.head_dim))


def _mutant_layer_step(mut):
    def layer_step(dims, lw, x, pos, cache, layer, trace=None, act="f16"):
        w1, w2 = (lw.ln2, lw.ln1) if mut == "ln_swap" else (lw.ln1, lw.ln2)
        a = ref.f16(ref.rmsnorm(x, w1, dims.eps))
        y = ref.gemv(*lw.qkv, a)
        b = lw.bqkv.astype(F64)
        if mut == "bias_after_rope":
            q, k, v = _split(dims, y, mut)
            bq, bk, bv = _split(dims, b, mut)
            q, k, v = ref.rope(q, pos, dims.theta) + bq, ref.rope(k, pos, dims.theta) + bk, v + bv
        else:
            q, k, v = _split(dims, y + b, mut)
            q, k = ref.rope(q, pos, dims.theta), ref.rope(k, pos, dims.theta)
        q, k, v = ref.f16(q), ref.f16(k), ref.f16(v)
        if mut == "attn_before_append" and pos > 0:
            o = ref.paged_attention(q, cache.k[layer], cache.v[layer], cache.page_table, pos,
                                    1.0 / np.sqrt(dims.head_dim), dims.page)
            cache.store(layer, pos, k, v)
        else:
            cache.store(layer, pos, k, v)
            o = ref.paged_attention(q, cache.k[layer], cache.v[layer], cache.page_table, pos + 1,
                                    1.0 / np.sqrt(dims.head_dim), dims.page)
        o = ref.f16(o).reshape(-1)
        x = ref.gemv(*lw.o, o) if mut == "no_attn_residual" else x + ref.gemv(*lw.o, o)
        a2 = ref.f16(ref.rmsnorm(x, w2, dims.eps))
        mi = a if mut == "mlp_reads_a" else a2
        h = ref.f16(ref.swiglu(ref.gemv(*lw.gate, mi), ref.gemv(*lw.up, mi)))
        return ref.gemv(*lw.down, h) if mut == "no_mlp_residual" else x + ref.gemv(*lw.down, h)
    return layer_step


def _mutant_forward(mut):
    def forward_teacher_forced(dims, layers, glob, tokens, out_positions, progress=None, act="f16"):
        get = layers if callable(layers) else layers.__getitem__
        tokens = np.asarray(tokens)
        T = len(tokens)
        pos = np.arange(T)
        X = glob.embed[tokens].astype(F64)
        scale = 1.0 / np.sqrt(dims.head_dim)
        for layer in range(dims.n_layers):
            lw = get(layer)
            w1, w2 = (lw.ln2, lw.ln1) if mut == "ln_swap" else (lw.ln1, lw.ln2)
            A = ref.f16(ref.rmsnorm(X, w1, dims.eps))
            Y = ref.gemv(*lw.qkv, A)
            b = lw.bqkv.astype(F64)
            if mut == "bias_after_rope":
                Q, K, V = _split(dims, Y, mut)
                bq, bk, bv = _split(dims, b, mut)
                Q, K, V = ref.rope(Q, pos, dims.theta) + bq, ref.rope(K, pos, dims.theta) + bk, V + bv
            else:
                Q, K, V = _split(dims, Y + b, mut)
                Q, K = ref.rope(Q, pos, dims.theta), ref.rope(K, pos, dims.theta)
            Q, K, V = ref.f16(Q), ref.f16(K), ref.f16(V)
            if mut == "attn_before_append":
                # position p sees 0..p-1 only (position 0 sees itself)
                grp = dims.n_q_heads // dims.n_kv_heads
                O = np.empty((T, dims.n_q_heads, dims.head_dim))
                for p in range(T):
                    lo = max(p, 1)
                    for h in range(dims.n_q_heads):
                        j = h // grp
                        w = ref.softmax((K[:lo, j].astype(F64) @ Q[p, h].astype(F64)) * scale)
                        O[p, h] = w @ V[:lo, j].astype(F64)
            else:
                O = ref.causal_attention(Q, K, V, scale)
            O = ref.f16(O).reshape(T, -1)
            X = ref.gemv(*lw.o, O) if mut == "no_attn_residual" else X + ref.gemv(*lw.o, O)
            A2 = ref.f16(ref.rmsnorm(X, w2, dims.eps))
            MI = A if mut == "mlp_reads_a" else A2
            H = ref.f16(ref.swiglu(ref.gemv(*lw.gate, MI), ref.gemv(*lw.up, MI)))
            X = ref.gemv(*lw.down, H) if mut == "no_mlp_residual" else X + ref.gemv(*lw.down, H)
        idx = np.asarray(out_positions)
        XF = ref.f16(ref.rmsnorm(X[idx], glob.lnf, dims.eps)).astype(F64)
        return XF @ glob.lm_head.astype(F64).T
    return forward_teacher_forced


LAYER_PINS = [lpins.test_hand_model_single_position_closed_form,
              lpins.test_hand_model_two_positions_rope_after_bias_closed_form]


@pytest.mark.parametrize("mut", WIRING)
@pytest.mark.parametrize("path", ["layer_step", "forward_teacher_forced"])
def test_planted_wiring_mistake_is_caught(monkeypatch, mut, path):
    """Planted in one path at a time: a pin must fail on that path alone."""
    if path == "layer_step":
        monkeypatch.setattr(ref, "layer_step", _mutant_layer_step(mut))
    else:
        monkeypatch.setattr(ref, "forward_teacher_forced", _mutant_forward(mut))
        monkeypatch.setattr(oracle, "forward_teacher_forced", ref.forward_teacher_forced)
    failed = 0
    for t in LAYER_PINS:
        try:
            t()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"wiring mistake {mut} in {path} passed every layer pin"


def test_unmutated_copies_pass_the_pins(monkeypatch):
    """The mutant harness itself is faithful: with no mistake planted, its
    copies of both paths pass the pins (so a caught mutant is the mistake)."""
    monkeypatch.setattr(ref, "layer_step", _mutant_layer_step(None))
    monkeypatch.setattr(ref, "forward_teacher_forced", _mutant_forward(None))
    monkeypatch.setattr(oracle, "forward_teacher_forced", ref.forward_teacher_forced)
    for t in LAYER_PINS:
        t()
