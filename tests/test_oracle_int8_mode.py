"""Pins of the oracle's int8-activation step mode (act="int8"): the pages'
integer path ([TS] "Engineering Challenges" item 3; [SP] "Three Critical
Engineering Challenges" item 3), in which every int4 GEMV input is quantised
per group of 128 before the integer dot products.

act_int8 is checked against quantize_act_int8 (pinned in test_oracle_pins)
and against the properties of round-to-nearest codes at scale max|x| / 127;
the layer's wiring (which four inputs are quantised) against gemv_w4a8 of
quantize_act_int8 on the traced fp16 inputs, with planted mistakes that must
fail; the batched teacher-forced pass against the sequential steps."""
import numpy as np
import pytest

import oracle
from oracle import ref
import synth

RNG = np.random.default_rng(2024)


def _vectors():
    x = RNG.standard_normal((5, 384)).astype(np.float16)
    x[1, 128:256] = 0                                 # an all-zero group
    x[2] *= np.float16(300)                           # large values (h-like)
    x[3, :128] = np.float16(1e-5)                     # subnormal-range group
    return x


def test_act_int8_is_quantize_act_int8_dequantised():
    x = _vectors()
    got = oracle.act_int8(x)
    for r in range(x.shape[0]):
        c, s = oracle.quantize_act_int8(x[r])
        want = c.astype(np.float64) * np.repeat(s.astype(np.float64), 128)
        assert np.array_equal(got[r], want), f"row {r}"
        assert np.array_equal(oracle.act_int8(x[r]), want)


def test_act_int8_codes_are_round_to_nearest_at_max_over_127():
    x = _vectors()
    d = oracle.act_int8(x)
    xg = x.astype(np.float64).reshape(5, 3, 128)
    dg = d.reshape(5, 3, 128)
    for r in range(5):
        for g in range(3):
            amax = np.max(np.abs(xg[r, g]))
            if amax == 0:
                assert np.all(dg[r, g] == 0)
                continue
            s = float(np.float32(np.float32(amax) / np.float32(127)))
            codes = dg[r, g] / s
            assert np.array_equal(codes, np.round(codes)), "codes are integers"
            assert np.max(np.abs(codes)) == 127, "the largest element maps to +-127"
            # half a step, plus the float32 quotient's own rounding
            assert np.max(np.abs(dg[r, g] - xg[r, g])) <= s / 2 * (1 + 2.0 ** -20)


def _tiny():
    dims = synth.TINY
    layers = [synth.layer_weights(dims, l, cfg=140) for l in range(dims.n_layers)]
    glob = synth.global_weights(dims, cfg=140)
    return dims, layers, glob


def _wiring_errors(dims, layers, glob, n_pos=3):
    """Largest relative mismatch between the int8-mode layer's traced GEMV
    results and gemv_w4a8 of quantize_act_int8 of its traced fp16 inputs."""
    cache = ref.KVCache(dims, 4, np.arange(4, dtype=np.int32))
    toks = synth.prompt_ids(dims, n_pos, cfg=140)
    worst = 0.0

    def w4a8(w, v):
        c, s = oracle.quantize_act_int8(v)
        return oracle.gemv_w4a8(*w, c, s)

    def rel(a, b):
        return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))

    for pos in range(n_pos):
        x = glob.embed[int(toks[pos])].astype(np.float64)
        for layer in range(dims.n_layers):
            lw = layers[layer]
            tr = {}
            x_new = ref.layer_step(dims, lw, x, pos, cache, layer, trace=tr, act="int8")
            worst = max(worst,
                        rel(tr["qkv"], w4a8(lw.qkv, tr["a"]) + lw.bqkv.astype(np.float64)),
                        rel(tr["x1"] - x, w4a8(lw.o, tr["o"])),
                        rel(tr["g"], w4a8(lw.gate, tr["a2"])),
                        rel(tr["u"], w4a8(lw.up, tr["a2"])),
                        rel(x_new - tr["x1"], w4a8(lw.down, tr["h"])))
            x = x_new
    return worst


def test_int8_layer_quantises_every_gemv_input():
    dims, layers, glob = _tiny()
    assert _wiring_errors(dims, layers, glob) < 1e-12


@pytest.mark.parametrize("skip", [0, 1, 2, 3, 4])
def test_planted_int8_wiring_mistake_is_caught(monkeypatch, skip):
    """A layer that leaves one of its five GEMV inputs (qkv, o, gate, up,
    down, in call order) unquantised fails the wiring pin."""
    calls = {"n": 0}

    def mutant(act):
        def f(v):
            i = calls["n"] % 5
            calls["n"] += 1
            return v if i == skip else oracle.act_int8(v)
        return f if act == "int8" else (lambda v: v)

    monkeypatch.setattr(ref, "_gemv_input", mutant)
    dims, layers, glob = _tiny()
    assert _wiring_errors(dims, layers, glob, n_pos=1) > 1e-6


def test_int8_forward_matches_sequential_steps():
    dims, layers, glob = _tiny()
    toks = synth.prompt_ids(dims, 20, cfg=141)
    positions = np.array([0, 7, 16, 19])
    batched = oracle.forward_teacher_forced(dims, layers, glob, toks, positions, act="int8")
    cache = ref.KVCache(dims, 4, np.array([2, 0, 3, 1], dtype=np.int32))
    out = {}
    for p in range(20):
        lg = oracle.decode_step(dims, layers, glob, cache, int(toks[p]), p, act="int8")
        if p in positions:
            out[p] = lg
    seq = np.stack([out[p] for p in positions])
    assert np.max(np.abs(batched - seq)) <= 1e-9 * max(1.0, float(np.max(np.abs(seq))))
    # the integer path is a different function of the weights: not the fp16 logits
    f16 = oracle.forward_teacher_forced(dims, layers, glob, toks, positions)
    assert np.max(np.abs(f16 - batched)) > 1e-4
