"""Pins that tie the CPU oracle to something other than itself.

Each test checks the oracle against an exact computation, a closed form, an
invariant the mathematics fixes, or a constant the source pages state.  They
are chosen so that a plausible slip (wrong group index, transposed operand,
wrong RoPE pairing or sign, wrong GQA grouping, eps outside the root, scale
missing, gate/up swapped, page table ignored) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _exact_f16(bits: np.ndarray):
    """Integer decomposition of fp16 bit patterns: value = sign * mant * 2**exp."""
    bits = bits.astype(np.int64)
    sign = np.where(bits >> 15, -1, 1)
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    mant = np.where(e > 0, m + 1024, m)
    exp = np.where(e > 0, e, 1) - 25
    return sign, mant, exp


# ---------------------------------------------------------------- dequant ---

def test_deq_exhaustive_exact():
    """Every code in [-8, 7] times every finite fp16 scale: deq is exact.

    The reference value is built from integers only (code * mantissa, then a
    power of two), independent of floating-point multiplication.
    """
    bits = np.arange(65536, dtype=np.uint32)
    finite = ((bits >> 10) & 0x1F) != 0x1F
    bits = bits[finite]
    assert bits.size == 63488
    s = bits.astype(np.uint16).view(np.float16).reshape(496, 128)      # one scale per group
    codes = np.tile(np.arange(-8, 8, dtype=np.int8), 8)                # 128 codes per group
    q = np.tile(codes, (496, 128))                                      # [496, 128*128]
    w = oracle.deq(q, s)
    sign, mant, exp = _exact_f16(bits.reshape(496, 128))
    qq = q.reshape(496, 128, 128).astype(np.int64)
    exact = np.ldexp((qq * (sign * mant)[:, :, None]).astype(np.float64),
                     np.broadcast_to(exp[:, :, None], qq.shape))
    assert np.array_equal(w.reshape(496, 128, 128), exact)
    # the fp32 product is exact too (<= 15 significant bits)
    w32 = q.astype(np.float32) * np.repeat(s.astype(np.float32), 128, axis=1)
    assert np.array_equal(w32.astype(np.float64), w)
    # rational spot check
    r = np.random.default_rng(5)
    for _ in range(300):
        n, k = int(r.integers(496)), int(r.integers(16384))
        ref = Fraction(int(q[n, k])) * Fraction(float(s[n, k // 128]))
        assert Fraction(float(w[n, k])) == ref


def test_deq_group_indexing():
    """One-hot x picks q[n,k] * s[n, k // 128]; constant codes sum the scales."""
    r = np.random.default_rng(1)
    n, k = 5, 512
    q = r.integers(-8, 8, (n, k), dtype=np.int8)
    s = (r.random((n, k // 128)) + 0.5).astype(np.float16)
    for kk in (0, 127, 128, 300, 511):
        x = np.zeros(k, np.float16)
        x[kk] = 1
        y = oracle.gemv(q, s, x)
        want = [int(q[i, kk]) * float(s[i, kk // 128]) for i in range(n)]
        assert list(y) == want
    ones = np.ones((n, k), np.int8)
    y = oracle.gemv(ones, s, np.ones(k, np.float16))
    assert np.array_equal(y, 128.0 * s.astype(np.float64).sum(axis=1))


def test_gemv_rational_bruteforce():
    """fp64 oracle within a few ulps of the exact rational sum (tiny and config-0 rows)."""
    r = np.random.default_rng(2)
    q, s, x = synth.gemv_case(4, 256, cfg=90)
    cases = [(q, s, x, range(4))]
    q0, s0, x0 = synth.gemv_cfg0()
    cases.append((q0, s0, x0, (0, 1791, 3583)))
    for q, s, x, rows in cases:
        y = oracle.gemv(q, s, x)
        xf = [Fraction(float(v)) for v in x]
        for n in rows:
            exact = Fraction(0)
            mag = Fraction(0)
            for kk in range(q.shape[1]):
                t = Fraction(int(q[n, kk])) * Fraction(float(s[n, kk // 128])) * xf[kk]
                exact += t
                mag += abs(t)
            err = abs(Fraction(float(y[n])) - exact)
            assert err <= mag * Fraction(1, 2 ** 44), (n, float(err))


# ------------------------------------------------- fp16 -> int4 quantiser ---

def _round_f16(fr: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a rational to binary16 (by bracketing)."""
    if fr == 0:
        return Fraction(0)
    c = np.float16(float(fr))
    cands = [np.nextafter(c, np.float16(-np.inf)), c, np.nextafter(c, np.float16(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - fr),
                                     int(np.array(v, np.float16).view(np.uint16)) & 1))
    return Fraction(float(best))


def test_quantize_int4_rational_bruteforce():
    """Scales and codes equal the quantiser's definition in exact rationals
    with one explicit fp16 rounding (groups of several magnitudes, fp16
    subnormals, the largest fp16, a zero group and a group whose scale
    underflows to zero)."""
    r = np.random.default_rng(13)
    w = (r.standard_normal((3, 4 * 128)) * np.repeat([0.02, 1e-5, 500.0, 1.0], 128)).astype(np.float16)
    w[1, 300] = np.float16(65504.0)
    w[2, 0:128] = 0
    w[2, 128:256] = np.float16(6e-8)                     # max/7 rounds to zero in fp16
    # exact ties: scale 1/16 (max 7/16), elements (k + 1/2) / 16 and their negatives
    ties = np.array([(k + 0.5) / 16 for k in range(-7, 7)], np.float64)
    w[2, 256:384] = np.resize(np.concatenate([ties, [7 / 16]]), 128).astype(np.float16)
    codes, scales = oracle.quantize_int4(w)
    assert codes.dtype == np.int8 and scales.dtype == np.float16
    for n in range(3):
        for g in range(4):
            ws = [Fraction(float(v)) for v in w[n, g * 128:(g + 1) * 128]]
            sc = _round_f16(max(abs(v) for v in ws) / 7)
            assert Fraction(float(scales[n, g])) == sc, (n, g)
            for i, v in enumerate(ws):
                want = 0 if sc == 0 else max(-8, min(7, _round_half_even(v / sc)))
                assert int(codes[n, g * 128 + i]) == want, (n, g, i)


def test_quantize_int4_bounds():
    """|w - code * scale| <= scale / 2 except where a code is clamped at -8..7,
    and every group's largest magnitude maps to +-7 (or clamps from 8)."""
    w = synth.normal_f16(np.random.default_rng(14), (16, 1024), scale=0.02)
    codes, scales = oracle.quantize_int4(w)
    s64 = np.repeat(scales.astype(np.float64), 128, axis=1)
    err = np.abs(w.astype(np.float64) - codes * s64)
    assert np.all(err <= s64 * 0.5 * (1 + 2 ** -10) + 1e-300)
    am = np.argmax(np.abs(w.astype(np.float64)).reshape(16, 8, 128), axis=2)
    top = np.abs(codes.reshape(16, 8, 128))[np.arange(16)[:, None], np.arange(8)[None, :], am]
    assert np.all(top == 7)


# ------------------------------------------------ int8 activations (W4A8) ---

def _round_f32(fr: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a rational to binary32 (by bracketing)."""
    if fr == 0:
        return Fraction(0)
    c = np.float32(float(fr))
    lo, hi = np.nextafter(c, np.float32(-np.inf)), np.nextafter(c, np.float32(np.inf))
    best = None
    for cand in (lo, c, hi):
        d = abs(Fraction(float(cand)) - fr)
        key = (d, int(np.array(cand, np.float32).view(np.uint32)) & 1)   # ties: even mantissa
        if best is None or key < best[0]:
            best = (key, cand)
    return Fraction(float(best[1]))


def _round_half_even(fr: Fraction) -> int:
    f = math.floor(fr)
    rem = fr - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def test_quantize_act_rational_bruteforce():
    """Scales and codes equal the quantiser's definition evaluated in exact
    rationals with explicit float32 roundings (groups of several magnitudes,
    fp16 subnormals and a group that is all zero)."""
    r = np.random.default_rng(11)
    x = (r.standard_normal(4 * 128) * np.repeat([1.0, 1e-3, 300.0, 1e-6], 128)).astype(np.float16)
    x[256 + 5] = np.float16(-65504.0)          # the largest magnitude fp16
    # exact ties: max 127/128 gives scale 2^-7, elements (k + 1/2) / 128
    ties = np.array([(k + 0.5) / 128 for k in range(-126, 126, 2)], np.float64)
    tg = np.resize(np.concatenate([ties, [127 / 128]]), 128).astype(np.float16)
    x = np.concatenate([x, np.zeros(128, np.float16), tg])
    codes, scales = oracle.quantize_act_int8(x)
    assert codes.dtype == np.int8 and scales.dtype == np.float32
    for g in range(len(x) // 128):
        xs = [Fraction(float(v)) for v in x[g * 128:(g + 1) * 128]]
        amax = max(abs(v) for v in xs)
        sc = _round_f32(amax / 127)
        assert Fraction(float(scales[g])) == sc, g
        for i, v in enumerate(xs):
            want = 0 if sc == 0 else max(-127, min(127, _round_half_even(_round_f32(v / sc))))
            assert int(codes[g * 128 + i]) == want, (g, i)


def test_quantize_act_bounds_and_extremes():
    """|x - code * scale| <= scale / 2 (plus the float32 quotient's rounding),
    the largest magnitude of a group maps to +-127, zero groups stay zero."""
    x = synth.gemv_cfg0()[2]
    codes, scales = oracle.quantize_act_int8(x)
    xr = codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 128)
    err = np.abs(x.astype(np.float64) - xr)
    assert np.all(err <= np.repeat(scales.astype(np.float64), 128) * (0.5 + 2 ** -20))
    xg = np.abs(x.astype(np.float64)).reshape(-1, 128)
    cg = np.abs(codes.astype(np.int64)).reshape(-1, 128)
    assert np.all(cg[np.arange(len(cg)), np.argmax(xg, axis=1)] == 127)
    assert np.all(cg <= 127)
    z, zs = oracle.quantize_act_int8(np.zeros(256, np.float16))
    assert np.all(z == 0) and np.all(zs == 0)


def test_gemv_w4a8_rational_and_reduces_to_w4a16():
    """The W4A8 GEMV is the exact rational sum of code * scale * code * scale
    (within fp64 rounding), and equals the W4A16 GEMV when the activations are
    exactly code * power-of-two scale."""
    q, s, x = synth.gemv_case(4, 384, cfg=91)
    xq, xs = oracle.quantize_act_int8(x)
    y = oracle.gemv_w4a8(q, s, xq, xs)
    for n in range(4):
        exact, mag = Fraction(0), Fraction(0)
        for kk in range(384):
            t = (Fraction(int(q[n, kk])) * Fraction(float(s[n, kk // 128])) *
                 Fraction(int(xq[kk])) * Fraction(float(xs[kk // 128])))
            exact += t
            mag += abs(t)
        assert abs(Fraction(float(y[n])) - exact) <= mag * Fraction(1, 2 ** 44)
    r = np.random.default_rng(12)
    codes = r.integers(-127, 128, 384)
    codes[::128] = 127                                           # every group reaches 127
    scale = np.repeat([2.0 ** -7, 2.0 ** -3, 2.0 ** -10], 128)
    xe = (codes * scale).astype(np.float16)
    assert np.array_equal(xe.astype(np.float64), codes * scale)   # exactly representable
    xq2, xs2 = oracle.quantize_act_int8(xe)
    assert np.array_equal(xq2.astype(np.int64), codes)
    assert np.array_equal(oracle.gemv_w4a8(q, s, xq2, xs2), oracle.gemv(q, s, xe))


# ------------------------------------------------------------------- glue ---

def test_rmsnorm_closed_forms():
    d = 64
    w = np.linspace(0.5, 1.5, d).astype(np.float16)
    # constant vector c*1: w * c / sqrt(c^2 + eps) -- pins eps inside the root
    for c in (1e-3, 0.5, 3.0):
        out = oracle.rmsnorm(np.full(d, c), w, 1e-6)
        want = w.astype(np.float64) * c / math.sqrt(c * c + 1e-6)
        assert np.allclose(out, want, rtol=1e-14, atol=0)
    assert abs(oracle.rmsnorm(np.full(d, 1e-3), np.ones(d), 1e-6)[0] - 1 / math.sqrt(2)) < 1e-12
    x = np.random.default_rng(3).standard_normal(d)
    a, b = oracle.rmsnorm(x, w), oracle.rmsnorm(8.0 * x, w)
    assert np.allclose(a, b, rtol=1e-6)
    # unit weights give a vector of RMS ~1
    z = oracle.rmsnorm(x, np.ones(d), 0.0)
    assert abs(np.sqrt(np.mean(z * z)) - 1.0) < 1e-12


def test_rope_closed_forms():
    D = 128
    e = np.eye(D)[None]          # [1 head? no: treat rows as heads] -> [1, D, D]
    e = np.eye(D)                # heads = D unit vectors
    # position 0 is the identity
    assert np.array_equal(oracle.rope(e, 0, 1e6), e)
    p = 7
    r = oracle.rope(e, p, 1e6)
    # pair (0, 64) turns by angle p; half-split pairing and sign convention
    assert np.allclose(r[0], np.cos(p) * e[0] + np.sin(p) * e[64], atol=1e-15)
    assert np.allclose(r[64], -np.sin(p) * e[0] + np.cos(p) * e[64], atol=1e-15)
    # pair (32, 96): frequency theta^(-64/128) = 1e-3, so position 1000 turns by 1 radian
    r = oracle.rope(e, 1000, 1e6)
    assert np.allclose(r[32], math.cos(1.0) * e[32] + math.sin(1.0) * e[96], atol=1e-12)
    # pair (63, 127): frequency 1e6^(-126/128)
    f = 1e6 ** (-126 / 128)
    assert np.allclose(r[63], math.cos(1000 * f) * e[63] + math.sin(1000 * f) * e[127], atol=1e-12)


def test_rope_invariants():
    g = np.random.default_rng(4)
    q = g.standard_normal((3, 128))
    k = g.standard_normal((3, 128))
    for p in (1, 17, 511, 8191):
        rq = oracle.rope(q, p)
        # each pair keeps its norm
        n0 = q[:, :64] ** 2 + q[:, 64:] ** 2
        n1 = rq[:, :64] ** 2 + rq[:, 64:] ** 2
        assert np.allclose(n0, n1, rtol=1e-12)
    # <R_p q, R_p' k> depends only on p - p'
    a = np.sum(oracle.rope(q, 40) * oracle.rope(k, 13), axis=-1)
    b = np.sum(oracle.rope(q, 540) * oracle.rope(k, 513), axis=-1)
    assert np.allclose(a, b, rtol=1e-9)
    # batched positions agree with per-position calls
    Z = g.standard_normal((5, 2, 128))
    pos = np.array([0, 3, 16, 100, 639])
    batched = oracle.rope(Z, pos)
    for i, pp in enumerate(pos):
        assert np.array_equal(batched[i], oracle.rope(Z[i], pp))


def test_swiglu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 0.7310585786300049) < 1e-15
    assert abs(oracle.silu(-30.0)) < 1e-11
    assert abs(oracle.silu(40.0) - 40.0) < 1e-14
    # gate goes through silu, up does not
    assert abs(oracle.swiglu(2.0, 3.0) - 3.0 * 2.0 / (1 + math.exp(-2.0))) < 1e-14
    assert oracle.swiglu(0.0, 5.0) == 0.0
    assert oracle.swiglu(5.0, 0.0) == 0.0


# -------------------------------------------------------------- attention ---

def test_softmax_sums_to_one():
    g = np.random.default_rng(6)
    for n in (1, 2, 17, 640, 8193):
        w = oracle.softmax(g.standard_normal(n) * 30)
        assert abs(w.sum() - 1.0) <= n * 2 ** -52
        assert (w >= 0).all()


def _pools(n_pages, n_kvh, D=128, seed=0):
    g = np.random.default_rng(seed)
    k = g.standard_normal((n_pages, n_kvh, 16, D)).astype(np.float16)
    v = g.standard_normal((n_pages, n_kvh, 16, D)).astype(np.float16)
    return k, v


def test_attention_one_token_returns_v_row():
    k, v = _pools(3, 4)
    q = np.random.default_rng(7).standard_normal((28, 128)).astype(np.float16)
    table = np.array([2, 0, 1], np.int32)
    o = oracle.paged_attention(q, k, v, table, 1, 1 / math.sqrt(128))
    for h in range(28):
        assert np.array_equal(o[h], v[2, h // 7, 0].astype(np.float64))


def test_attention_gqa_mapping():
    """Heads 7j..7j+6 read kv head j (consecutive grouping, not h mod 4)."""
    k, v = _pools(1, 4)
    for j in range(4):
        v[0, j, :3] = j + 1           # every token of kv head j has V = j+1
    q = np.random.default_rng(8).standard_normal((28, 128)).astype(np.float16)
    o = oracle.paged_attention(q, k, v, np.array([0], np.int32), 3, 0.1)
    for h in range(28):
        assert np.allclose(o[h], h // 7 + 1, rtol=0, atol=1e-15)


def test_attention_two_token_closed_form():
    """Weights are sigmoid(+-(s1-s2)) with s = q.k / sqrt(128)."""
    k, v = _pools(1, 1)
    q = np.zeros((1, 128), np.float16)
    q[0, 0] = 8
    k[0, 0, 0] = 0
    k[0, 0, 0, 0] = 8          # s1 = 64 / sqrt(128)
    k[0, 0, 1] = 0             # s2 = 0
    o = oracle.paged_attention(q, k, v, np.array([0], np.int32), 2, 1 / math.sqrt(128))
    w1 = 1.0 / (1.0 + math.exp(-64 / math.sqrt(128)))
    want = w1 * v[0, 0, 0].astype(np.float64) + (1 - w1) * v[0, 0, 1].astype(np.float64)
    assert np.allclose(o[0], want, rtol=0, atol=1e-14)


def test_attention_equal_keys_mean_of_v():
    k, v = _pools(2, 1)
    k[:] = k[0, 0, 0]
    q = np.random.default_rng(9).standard_normal((2, 128)).astype(np.float16)
    o = oracle.paged_attention(q, k, v, np.array([1, 0], np.int32), 29, 0.3)
    vals = np.concatenate([v[1, 0], v[0, 0, :13]]).astype(np.float64)
    assert np.allclose(o, vals.mean(axis=0), rtol=0, atol=1e-13)


def test_attention_page_table_shuffle_invariance_and_tail():
    q, kp, vp, table = synth.attn_case(37, n_qh=28, n_kvh=4, n_pages=5, cfg=91)
    ctx = 37
    o = oracle.paged_attention(q, kp, vp, table, ctx, 1 / math.sqrt(128))
    # the same tokens laid out contiguously give the identical result
    kc = np.zeros_like(kp)
    vc = np.zeros_like(vp)
    for i, ph in enumerate(table):
        kc[i], vc[i] = kp[ph], vp[ph]
    o2 = oracle.paged_attention(q, kc, vc, np.arange(len(table), dtype=np.int32), ctx,
                                1 / math.sqrt(128))
    assert np.array_equal(o, o2)
    # slots past ctx in the last page, and unused pages, are never read
    kp2, vp2 = kp.copy(), vp.copy()
    last = table[ctx // 16]
    kp2[last, :, ctx % 16:] = np.float16(60000)
    vp2[last, :, ctx % 16:] = np.float16(np.nan)
    for ph in set(range(5)) - set(table.tolist()):
        vp2[ph] = np.float16(np.nan)
    o3 = oracle.paged_attention(q, kp2, vp2, table, ctx, 1 / math.sqrt(128))
    assert np.array_equal(o, o3)


def test_causal_attention_matches_paged():
    g = np.random.default_rng(10)
    T = 35
    Q = g.standard_normal((T, 4, 128)).astype(np.float16)
    K = g.standard_normal((T, 2, 128)).astype(np.float16)
    V = g.standard_normal((T, 2, 128)).astype(np.float16)
    O = oracle.causal_attention(Q, K, V, 0.2)
    kp = np.zeros((3, 2, 16, 128), np.float16)
    vp = np.zeros_like(kp)
    table = np.array([2, 0, 1], np.int32)
    for t in range(T):
        kp[table[t // 16], :, t % 16] = K[t]
        vp[table[t // 16], :, t % 16] = V[t]
    for p in (0, 15, 16, 34):
        o = oracle.paged_attention(Q[p], kp, vp, table, p + 1, 0.2)
        assert np.allclose(o, O[p], rtol=0, atol=1e-13)


# ------------------------------------------------------------------ model ---

def test_argmax_lowest_index():
    assert oracle.argmax_first(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert oracle.argmax_first(np.array([5.0])) == 0


def _tiny_model(zero_codes=False):
    dims = synth.TINY
    layers = [synth.layer_weights(dims, l, cfg=92) for l in range(dims.n_layers)]
    glob = synth.global_weights(dims, cfg=92)
    if zero_codes:
        for lw in layers:
            for name in ("qkv", "o", "gate", "up", "down"):
                qq, ss = getattr(lw, name)
                setattr(lw, name, (np.zeros_like(qq), ss))
    return dims, layers, glob


def test_zero_projection_model_reduces_to_one_matmul():
    """All projection codes 0: the residual stays E[t]; logits = W_lm f16(norm(E[t]) w_f)."""
    dims, layers, glob = _tiny_model(zero_codes=True)
    n_pages = 4
    cache = oracle.KVCache(dims, n_pages, np.arange(n_pages))
    toks = [3, 999, 0, 512]
    for p, t in enumerate(toks):
        logits = oracle.decode_step(dims, layers, glob, cache, t, p)
        e = glob.embed[t].astype(np.float64)
        xf = (e / np.sqrt(np.mean(e * e) + dims.eps) * glob.lnf.astype(np.float64)).astype(np.float16)
        want = glob.lm_head.astype(np.float64) @ xf.astype(np.float64)
        assert np.allclose(logits, want, rtol=1e-13, atol=1e-13)


def test_sequential_decode_equals_teacher_forced_pass():
    """Paged, shuffled sequential decode == contiguous batched pass (2 layers, 40 tokens)."""
    dims, layers, glob = _tiny_model()
    T = 40
    toks = synth.prompt_ids(dims, T, cfg=92)
    free = synth.page_free_list(4, cfg=92)
    cache = oracle.KVCache(dims, 4, free)
    seq = np.stack([oracle.decode_step(dims, layers, glob, cache, int(toks[p]), p)
                    for p in range(T)])
    bat = oracle.forward_teacher_forced(dims, layers, glob, toks, np.arange(T))
    assert np.allclose(seq, bat, rtol=1e-10, atol=1e-10)
    # the cache holds the pass's K rows at the free-list pages
    assert cache.k[0][free[2], 0, 5].any()


def test_printed_constants():
    c = json.load(open(os.path.join(GOLDEN, "printed_constants.json")))
    d = synth.QWEN7B
    assert d.n_layers == c["n_layers"]["value"]
    assert d.d_model == c["d_model"]["value"]
    assert d.d_ff == c["d_ff"]["value"]
    assert d.group == c["quant_group"]["value"]
    assert d.page == c["page_tokens"]["value"]
    kp = np.zeros((1, d.n_kv_heads, d.page, d.head_dim), np.float16)
    assert kp[0, 0].nbytes == c["kv_head_slice_bytes"]["value"]
    # the decode workload (512 prompt + 128 generated) ends at 40 pages of 16
    total = c["prompt_tokens"]["value"] + c["generated_tokens"]["value"]
    assert total // d.page == 40
