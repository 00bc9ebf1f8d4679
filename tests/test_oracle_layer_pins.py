"""Closed-form pins of the oracle's decoder-block composition.

The component pins (tests/test_oracle_pins.py) fix each op on its own; these
fix how a layer wires them: which norm weight feeds which projection, that
the QKV bias is added before RoPE, the q | k | v split order, that the new
token's K/V are appended before attention, that the MLP reads the
post-attention norm, and both residual adds.

A one-layer model of width 128 is built by hand so that every intermediate
can be written down: all group scales 1, one-hot ("identity") projections,
constant or sign-alternating embeddings (RMSNorm of x = c * (+-1) is +-1 up to
eps, so the normalised input is the norm weight itself, after the fp16
rounding), an identity lm_head (logits = the final normalised state).  The
expected values below follow the model's definition step by step on these
inputs ([TS] "Technical Specifications and Hardware Alignment" for the weight
set; softmax + weighted-V attention, [SP] "Three Critical Engineering
Challenges" item 1); each norm's mean of squares is taken exactly with
fractions, so no oracle routine is reused.

Both oracle paths are checked: the sequential paged decode (``decode_step``,
which runs ``layer_step``) and the batched teacher-forced pass
(``forward_teacher_forced``).  tests/test_oracle_mutants.py plants wiring
mistakes in both and checks that these pins catch each.
"""
import math
from fractions import Fraction

import numpy as np

import oracle
import synth

D = 128
DIMS = synth.ModelDims(d_model=D, d_ff=D, n_layers=1, n_q_heads=1, n_kv_heads=1,
                       head_dim=D, vocab=D)
ALPHA = 8.0      # q bias at dim 0
BETA = 8.0       # k bias at dim 0


def _f16(v: float) -> float:
    return float(np.float16(v))


def _ident(n, scale_code=1):
    q = np.zeros((n, D), np.int8)
    q[np.arange(n), np.arange(n) % D] = scale_code
    return q


def hand_model():
    """(layers, glob) of the hand-built one-layer model."""
    ones_s = lambda n: np.ones((n, 1), np.float16)   # noqa: E731  (one group per row, scale 1)
    k = np.arange(D)
    ln1 = (1.0 + k / 128).astype(np.float16)
    ln2 = (0.5 + k / 512).astype(np.float16)
    lnf = (1.5 - k / 256).astype(np.float16)
    qkv = np.zeros((3 * D, D), np.int8)
    qkv[2 * D + k, k] = 1                            # v = a; q and k rows all zero
    b = np.zeros(3 * D, np.float16)
    b[0] = ALPHA                                     # q from the bias alone
    b[D] = BETA                                      # k from the bias alone
    lw = synth.LayerWeights(
        ln1=ln1, qkv=(qkv, ones_s(3 * D)), bqkv=b,
        o=(_ident(D), ones_s(D)), ln2=ln2,
        gate=(_ident(D), ones_s(D)), up=(_ident(D, 2), ones_s(D)),
        down=(_ident(D), ones_s(D)))
    embed = np.zeros((D, D), np.float16)
    embed[0] = 2.0                                   # token 0: constant 2
    embed[1] = np.where(k % 2 == 0, 2.0, -2.0)       # token 1: +-2 alternating
    embed[2:] = 1.0
    glob = synth.GlobalWeights(embed=embed, lnf=lnf, lm_head=np.eye(D, dtype=np.float16))
    return [lw], glob


def _norm_scale(x):
    """1 / sqrt(mean(x^2) + eps), the mean of squares taken exactly."""
    ms = sum(Fraction(float(v)) ** 2 for v in x) / len(x)
    return 1.0 / math.sqrt(float(ms) + DIMS.eps)


def _normed(x, w):
    r = _norm_scale(x)
    return [_f16(float(xi) * r * float(wi)) for xi, wi in zip(x, w)]


def _after_attention(x_in, o, lw, glob):
    """From the residual entering the layer and the attention output: the
    final logits (O identity, residual, RMSNorm ln2, gate = a2 and up = 2 a2,
    SwiGLU, down identity, residual, final norm, identity lm_head)."""
    x1 = [xi + oi for xi, oi in zip(x_in, o)]
    a2 = _normed(x1, lw.ln2)
    h = [_f16(g * (2.0 * g) / (1.0 + math.exp(-g))) for g in a2]
    x2 = [xi + hi for xi, hi in zip(x1, h)]
    return np.array(_normed(x2, glob.lnf)), dict(x1=x1, a2=a2, h=h, x2=x2)


def expected_position0():
    """Token 0 at position 0 (context of one token)."""
    layers, glob = hand_model()
    lw = layers[0]
    x0 = [2.0] * D
    # RMSNorm of a constant 2: 2 / sqrt(4 + 1e-6) = 1 - 1.25e-7, far inside
    # half an fp16 ulp, so a is ln1 exactly
    a = [float(w) for w in lw.ln1]
    assert _normed(x0, lw.ln1) == a
    v = a                                            # v rows are the identity on a, no bias
    o = v                                            # one cached token: softmax weight 1
    logits, mid = _after_attention(x0, o, lw, glob)
    return logits, dict(a=a, v=v, o=o, **mid)


def expected_position1():
    """Token 1 at position 1, after token 0 at position 0.

    q and k come from the biases alone (ALPHA, BETA at dim 0); RoPE turns
    pair (0, 64) by angle 1 at position 1 and not at all at position 0.  So
    k0 = BETA e0 and q1 = k1 = (f16(8 cos 1), f16(8 sin 1)) on dims (0, 64).
    v0 = ln1 and v1 = sign * ln1 (the embedding of token 1 alternates in
    sign, so does its normalised input).  Two-token softmax:
    o = w0 v0 + w1 v1, w0 = 1 / (1 + exp(s1 - s0)).
    """
    layers, glob = hand_model()
    lw = layers[0]
    k = np.arange(D)
    sign = np.where(k % 2 == 0, 1.0, -1.0)
    x0 = list(2.0 * sign)
    a = [float(w) for w in lw.ln1 * sign.astype(np.float16)]
    assert _normed(x0, lw.ln1) == a
    c, s = _f16(ALPHA * math.cos(1.0)), _f16(ALPHA * math.sin(1.0))
    ck, sk = _f16(BETA * math.cos(1.0)), _f16(BETA * math.sin(1.0))
    scale = 1.0 / math.sqrt(D)
    s0 = c * BETA * scale                           # q1 . k0 (k0 unrotated at position 0)
    s1 = (c * ck + s * sk) * scale                  # q1 . k1
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    v0 = [float(w) for w in lw.ln1]
    v1 = a
    o = [_f16(w0 * p + w1 * q) for p, q in zip(v0, v1)]
    logits, mid = _after_attention(x0, o, lw, glob)
    return logits, dict(a=a, o=o, w0=w0, **mid)


TOL = 1e-12


def test_hand_model_single_position_closed_form():
    layers, glob = hand_model()
    want, mid = expected_position0()
    cache = oracle.KVCache(DIMS, 1, np.array([0]))
    got = oracle.decode_step(DIMS, layers, glob, cache, 0, 0)
    assert np.allclose(got, want, rtol=0, atol=TOL), float(np.max(np.abs(got - want)))
    # the new token's K and V rows are in the cache (physical page 0, slot 0)
    assert float(cache.k[0][0, 0, 0, 0]) == BETA and not cache.k[0][0, 0, 0, 1:].any()
    assert np.array_equal(cache.v[0][0, 0, 0].astype(np.float64), np.array(mid["v"]))
    tf = oracle.forward_teacher_forced(DIMS, layers, glob, np.array([0]), [0])
    assert np.allclose(tf[0], want, rtol=0, atol=TOL), float(np.max(np.abs(tf[0] - want)))


def test_hand_model_layer_trace_closed_form():
    """The intermediates layer_step reports match the hand derivation."""
    layers, glob = hand_model()
    _, mid = expected_position0()
    cache = oracle.KVCache(DIMS, 1, np.array([0]))
    tr = {}
    x = oracle.layer_step(DIMS, layers[0], glob.embed[0].astype(np.float64), 0, cache, 0, trace=tr)
    assert np.array_equal(tr["a"].astype(np.float64), np.array(mid["a"]))
    assert np.array_equal(tr["o"].astype(np.float64), np.array(mid["o"]))
    assert np.array_equal(tr["a2"].astype(np.float64), np.array(mid["a2"]))
    assert np.array_equal(tr["h"].astype(np.float64), np.array(mid["h"]))
    assert np.allclose(x, np.array(mid["x2"]), rtol=0, atol=TOL)
    assert float(tr["q"][0, 0]) == ALPHA and float(tr["k"][0, 0]) == BETA


def test_hand_model_two_positions_rope_after_bias_closed_form():
    layers, glob = hand_model()
    want0, _ = expected_position0()
    want1, mid = expected_position1()
    assert 0.01 < mid["w0"] < 0.2                    # far from the 1/2 that ignoring RoPE would give
    pt = np.array([0])
    cache = oracle.KVCache(DIMS, 1, pt)
    g0 = oracle.decode_step(DIMS, layers, glob, cache, 0, 0)
    g1 = oracle.decode_step(DIMS, layers, glob, cache, 1, 1)
    assert np.allclose(g0, want0, rtol=0, atol=TOL)
    assert np.allclose(g1, want1, rtol=0, atol=TOL), float(np.max(np.abs(g1 - want1)))
    tf = oracle.forward_teacher_forced(DIMS, layers, glob, np.array([0, 1]), [0, 1])
    assert np.allclose(tf[0], want0, rtol=0, atol=TOL)
    assert np.allclose(tf[1], want1, rtol=0, atol=TOL), float(np.max(np.abs(tf[1] - want1)))


def test_mlp_closed_form():
    """oracle.mlp with gate = identity, up = 2 x identity, down = identity:
    h = f16(silu(x) * 2x), y = h."""
    x = (np.linspace(-6, 6, D)).astype(np.float16)
    ones = np.ones((D, 1), np.float16)
    h, y = oracle.mlp(x, (_ident(D), ones), (_ident(D, 2), ones), (_ident(D), ones))
    want = np.array([_f16(float(v) * 2.0 * float(v) / (1.0 + math.exp(-float(v)))) for v in x])
    assert np.array_equal(h.astype(np.float64), want)
    assert np.array_equal(y, want)
    # a down projection that is not the identity: reversed rows
    dq = np.zeros((D, D), np.int8)
    dq[np.arange(D), D - 1 - np.arange(D)] = 3
    _, y2 = oracle.mlp(x, (_ident(D), ones), (_ident(D, 2), ones), (dq, ones))
    assert np.array_equal(y2, 3.0 * want[::-1])
