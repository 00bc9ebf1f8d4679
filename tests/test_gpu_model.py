"""Decode-step parity: the graph-captured GPU step against the oracle's
teacher-forced pass, graph == eager bitwise, page-table bookkeeping, and the
step's error paths."""
import json
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth
import int4_weight_only_dequant_amd as w4
from int4_weight_only_dequant_amd import _lib as L
from tests._tol import LOGIT_ATOL

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_model(model, prompt, n_steps, flags=L.W4_GRAPH):
    """Teacher-forced prompt, then free-running greedy steps; returns per-step
    logits (float32 [n_steps, V]) and the token history."""
    model.reset(prompt)
    out = []
    for _ in range(n_steps):
        model.step(flags)
        out.append(model.logits.clone())
    torch.cuda.synchronize()
    toks = model.tokens[: n_steps + 1].cpu().numpy()
    return torch.stack(out).cpu().numpy(), toks


_ORACLE_CACHE = {}


def compare_with_oracle(dims, layers, glob, logits, toks, n_prompt, positions, cache_key=None, act="f16"):
    """Worst |logit error| at positions and the greedy-token mismatches against
    the oracle in activation mode act: a differing token counts unless its
    oracle logit is within twice that position's logit error of the oracle's
    top-1 (a near tie, reported as such).  With cache_key, the oracle pass
    for the same key and token history is reused."""
    key = None if cache_key is None else (cache_key, act, toks[: positions[-1] + 1].tobytes(), positions.tobytes())
    ref = _ORACLE_CACHE.get(key) if key is not None else None
    if ref is None:
        ref = oracle.forward_teacher_forced(dims, layers, glob, toks[: positions[-1] + 1], positions,
                                            progress=lambda l: say(f"  oracle layer {l} done"), act=act)
        if key is not None:
            _ORACLE_CACHE[key] = ref
    err = np.abs(logits[positions] - ref)
    worst = float(err.max())
    mism = []
    ties = []
    margins = []
    for i, p in enumerate(positions):
        want = oracle.argmax_first(ref[i])
        srt = np.sort(ref[i])
        margin = float(srt[-1] - srt[-2])
        margins.append(margin)
        got = int(toks[p + 1])
        if p + 1 >= n_prompt and got != want:
            # logits within e of the oracle's can only reorder tokens whose
            # oracle logits are within 2 e: such a flip is a tie at the
            # measured precision, any other is a mismatch
            gap = float(ref[i][want] - ref[i][got])
            e_pos = float(err[i].max())
            (ties if gap <= 2 * e_pos else mism).append((int(p), got, want, gap))
    gen = toks[positions + 1]
    rec = {"act": act, "positions": f"{int(positions[0])}-{int(positions[-1])}", "max_logit_err": worst,
           "min_top2_margin": float(min(margins)), "distinct_generated_tokens": int(len(np.unique(gen))),
           "token_mismatches": len(mism), "near_tie_flips": ties}
    say(f"  parity record: {json.dumps(rec)}")
    if os.environ.get("W4_PARITY_REPORT"):
        with open(os.environ["W4_PARITY_REPORT"], "a") as fh:
            fh.write(json.dumps({"case": cache_key or "model", **rec}) + "\n")
    return worst, mism


@pytest.mark.parametrize("path", ["persistent", "multi"])
def test_tiny_model_parity_graph_eager_and_pages(path):
    dims = synth.TINY
    layers = [synth.layer_weights(dims, l, cfg=102) for l in range(dims.n_layers)]
    glob = synth.global_weights(dims, cfg=102)
    max_pages = 4
    free = synth.page_free_list(max_pages, cfg=102)
    prompt = synth.prompt_ids(dims, 20, cfg=102)
    extra = L.W4_MULTI if path == "multi" else 0
    say(f"case: tiny model (2 layers) {path} path, 20-token prompt + 44 steps, 4 shuffled pages")
    model = w4.DecodeModel(dims, lambda l: layers[l], glob, free, max_pages)
    try:
        say(f"  persistent grid {model.grid()} work-groups")
        n = 64
        lg, tk = run_model(model, prompt, n, L.W4_GRAPH | extra)
        assert model.device_error() == 0
        pt = model.page_table.cpu().numpy()
        assert np.array_equal(pt, free)                    # every boundary appended its page
        le, te = run_model(model, prompt, n, L.W4_EAGER | extra)
        assert model.device_error() == 0
        assert np.array_equal(tk, te)
        assert np.array_equal(lg.view(np.uint32), le.view(np.uint32))   # graph == eager bitwise
        assert np.array_equal(tk[:20], prompt)
        worst, mism = compare_with_oracle(dims, layers, glob, lg, tk, 20, np.arange(n))
        say(f"tiny {path}: max |logit err| {worst:.3e}; token mismatches {mism}")
        assert worst <= LOGIT_ATOL
        assert not mism
        # error paths
        with pytest.raises(w4.W4Error) as e:
            w4.decode_step(model, 3, L.W4_GRAPH)
        assert e.value.status == L.W4_ESTATE
        with pytest.raises(w4.W4Error) as e:
            model.step()                                   # position 64 = 16 * max_pages: pool full
        assert e.value.status == L.W4_ENOSPC
    finally:
        model.close()


def test_tiny_persistent_matches_multikernel():
    """Both step implementations on the same model agree closely (different
    summation orders, same fp16 storage points)."""
    dims = synth.TINY
    layers = [synth.layer_weights(dims, l, cfg=103) for l in range(dims.n_layers)]
    glob = synth.global_weights(dims, cfg=103)
    free = synth.page_free_list(4, cfg=103)
    prompt = synth.prompt_ids(dims, 40, cfg=103)
    say("case: tiny model persistent vs kernel-per-op, 40 prompt + 24 steps")
    model = w4.DecodeModel(dims, lambda l: layers[l], glob, free, 4)
    try:
        la, ta = run_model(model, prompt, 64, L.W4_GRAPH)
        lb, tb = run_model(model, prompt, 64, L.W4_GRAPH | L.W4_MULTI)
        assert model.device_error() == 0
    finally:
        model.close()
    diff = float(np.max(np.abs(la - lb)))
    say(f"persistent vs multi: max |logit diff| {diff:.3e}")
    assert diff <= 1e-2
    assert np.array_equal(ta, tb)


@pytest.mark.parametrize("n_qh,n_kvh", [(14, 2), (4, 2)])
def test_gqa_step_with_a_large_pool(n_qh, n_kvh):
    """GQA 7:1 and 2:1 on a 136-page pool (several attention chunks per head):
    280 teacher-forced + 20 greedy steps against the oracle."""
    dims = synth.ModelDims(d_model=512, d_ff=1024, n_layers=2, n_q_heads=n_qh, n_kv_heads=n_kvh,
                           head_dim=128, vocab=1000)
    layers = [synth.layer_weights(dims, l, cfg=122) for l in range(dims.n_layers)]
    glob = synth.global_weights(dims, cfg=122)
    max_pages = 136
    free = synth.page_free_list(max_pages, cfg=122)
    prompt = synth.prompt_ids(dims, 280, cfg=122)
    say(f"case: GQA {n_qh}/{n_kvh}, 136-page pool, 280 prompt + 20 steps")
    model = w4.DecodeModel(dims, lambda l: layers[l], glob, free, max_pages)
    try:
        lg, tk = run_model(model, prompt, 300)
        assert model.device_error() == 0
    finally:
        model.close()
    positions = np.arange(279, 300)
    worst, mism = compare_with_oracle(dims, layers, glob, lg, tk, 280, positions)
    say(f"  max |logit err| {worst:.3e}; mismatches {mism}")
    assert worst <= LOGIT_ATOL
    assert not mism


def test_tiny_model_from_container_equals_arrays(tmp_path):
    """A model loaded from the weight container (mapped, pre-packed tensors)
    steps bit-identically to the same model packed from arrays."""
    from int4_weight_only_dequant_amd import model as M
    dims = synth.TINY
    layers = [synth.layer_weights(dims, l, cfg=121) for l in range(dims.n_layers)]
    glob = synth.global_weights(dims, cfg=121)
    free = synth.page_free_list(4, cfg=121)
    prompt = synth.prompt_ids(dims, 20, cfg=121)
    path = str(tmp_path / "tiny.w4c")
    M.write_model_container(path, dims, lambda l: layers[l], glob)
    say("case: tiny model from container vs from arrays, 20 prompt + 12 steps")
    a = w4.DecodeModel(dims, lambda l: layers[l], glob, free, 4)
    try:
        la, ta = run_model(a, prompt, 32)
    finally:
        a.close()
    b = w4.DecodeModel.from_container(path, free, 4)
    try:
        lb, tb = run_model(b, prompt, 32)
        assert b.device_error() == 0
    finally:
        b.close()
    assert np.array_equal(la, lb) and np.array_equal(ta, tb)


@pytest.mark.slow
@pytest.mark.timeout(1500)
def test_full_model_512_plus_128():
    """The Qwen2.5-7B-shaped step: 512-token prompt, 128 greedy graph steps
    crossing 8 page boundaries; 129 logit vectors and tokens vs the oracle."""
    dims = synth.QWEN7B
    t0 = time.time()
    say("case: full model 28 layers, prompt 512 + 128 generated, 40 shuffled pages")
    glob = synth.global_weights(dims)
    free = synth.page_free_list(40)
    prompt = synth.prompt_ids(dims, 512)
    model = w4.DecodeModel(dims, lambda l: synth.layer_weights(dims, l), glob, free, 40,
                           progress=lambda l: say(f"  packed+uploaded layer {l} ({time.time() - t0:.0f}s)"))
    try:
        say(f"model ready {time.time() - t0:.0f}s")
        lg, tk = run_model(model, prompt, 640, L.W4_GRAPH)
        assert model.device_error() == 0
        pt = model.page_table.cpu().numpy()
    finally:
        model.close()
    say(f"GPU run done {time.time() - t0:.0f}s; tokens {tk[512:530]}...")
    assert np.array_equal(pt, free)
    positions = np.arange(511, 640)
    worst, mism = compare_with_oracle(dims, lambda l: synth.layer_weights(dims, l), glob, lg, tk,
                                      512, positions, cache_key="qwen7b-512+128")
    say(f"full: max |logit err| over 129 positions {worst:.3e}; mismatches {mism} ({time.time() - t0:.0f}s)")
    assert worst <= LOGIT_ATOL
    assert not mism


@pytest.mark.slow
@pytest.mark.timeout(1500)
def test_full_model_prefill_512_then_128_steps():
    """The same workload with the prompt taken by one 512-token prefill call
    (matrix-core GEMMs, causal paged attention), then 128 greedy graph steps
    on the cache it wrote; logits at positions 511..639 vs the oracle."""
    dims = synth.QWEN7B
    t0 = time.time()
    say("case: full model 28 layers, prefill 512 + 128 generated, 40 shuffled pages")
    glob = synth.global_weights(dims)
    free = synth.page_free_list(40)
    prompt = synth.prompt_ids(dims, 512)
    model = w4.DecodeModel(dims, lambda l: synth.layer_weights(dims, l), glob, free, 40,
                           progress=lambda l: say(f"  packed+uploaded layer {l} ({time.time() - t0:.0f}s)"))
    try:
        model.reset(prompt)
        model.prefill(512)
        out = [model.logits.clone()]
        for _ in range(128):
            model.step()
            out.append(model.logits.clone())
        torch.cuda.synchronize()
        assert model.device_error() == 0
        lg = torch.stack(out).cpu().numpy()
        tk = model.tokens[:641].cpu().numpy()
        pt = model.page_table.cpu().numpy()
    finally:
        model.close()
    say(f"GPU run done {time.time() - t0:.0f}s; tokens {tk[512:530]}...")
    assert np.array_equal(pt, free)
    positions = np.arange(511, 640)
    full = np.zeros((640, lg.shape[1]), np.float32)
    full[positions] = lg
    worst, mism = compare_with_oracle(dims, lambda l: synth.layer_weights(dims, l), glob, full, tk,
                                      512, positions, cache_key="qwen7b-512+128")
    say(f"prefill: max |logit err| over 129 positions {worst:.3e}; mismatches {mism} ({time.time() - t0:.0f}s)")
    assert worst <= LOGIT_ATOL
    assert not mism


# ------------------------------------------------- int8 activations (W4_A8) --

@pytest.mark.parametrize("dims_name", ["tiny", "gqa"])
def test_a8_step_parity_graph_eager(dims_name):
    """The int8-activation persistent step against the oracle's int8 mode
    (same tolerance as the fp16 step: the quantisation is the same function
    of the same fp16 inputs on both sides), graph == eager bitwise, and the
    flag's refusals."""
    if dims_name == "tiny":
        dims, n_prompt, n, max_pages = synth.TINY, 20, 64, 4
    else:
        dims = synth.ModelDims(d_model=512, d_ff=1024, n_layers=2, n_q_heads=14, n_kv_heads=2,
                               head_dim=128, vocab=1000)
        n_prompt, n, max_pages = 150, 180, 12
    layers = [synth.layer_weights(dims, l, cfg=150) for l in range(dims.n_layers)]
    glob = synth.global_weights(dims, cfg=150)
    free = synth.page_free_list(max_pages, cfg=150)
    prompt = synth.prompt_ids(dims, n_prompt, cfg=150)
    say(f"case: {dims_name} model, int8 activations, {n_prompt} prompt + {n - n_prompt} steps")
    model = w4.DecodeModel(dims, lambda l: layers[l], glob, free, max_pages)
    try:
        lg, tk = run_model(model, prompt, n, L.W4_GRAPH | L.W4_A8)
        assert model.device_error() == 0
        le, te = run_model(model, prompt, n, L.W4_EAGER | L.W4_A8)
        assert model.device_error() == 0
        assert np.array_equal(tk, te)
        assert np.array_equal(lg.view(np.uint32), le.view(np.uint32))
        lf, _ = run_model(model, prompt, n, L.W4_GRAPH)
        assert np.max(np.abs(lf - lg)) > 1e-4, "the int8 step differs from the fp16 step"
        model.reset(prompt)
        with pytest.raises(w4.W4Error) as e:
            model.step(L.W4_GRAPH | L.W4_A8 | L.W4_MULTI)
        assert e.value.status == L.W4_EINVAL
    finally:
        model.close()
    positions = np.arange(n_prompt - 1, n)
    worst, mism = compare_with_oracle(dims, layers, glob, lg, tk, n_prompt, positions, act="int8")
    say(f"  a8 {dims_name}: max |logit err| {worst:.3e}; mismatches {mism}")
    assert worst <= LOGIT_ATOL
    assert not mism


@pytest.mark.slow
@pytest.mark.timeout(1500)
def test_full_model_a8_64_plus_64():
    """The 7B-shaped int8-activation step: a 64-token prompt, 64 greedy graph
    steps (4 page boundaries), logits at positions 63..127 against the
    oracle's int8 mode."""
    dims = synth.QWEN7B
    t0 = time.time()
    say("case: full model 28 layers, int8 activations, prompt 64 + 64 generated, 8 shuffled pages")
    glob = synth.global_weights(dims)
    free = synth.page_free_list(8)
    prompt = synth.prompt_ids(dims, 64)
    model = w4.DecodeModel(dims, lambda l: synth.layer_weights(dims, l), glob, free, 8,
                           progress=lambda l: say(f"  packed+uploaded layer {l} ({time.time() - t0:.0f}s)"))
    try:
        lg, tk = run_model(model, prompt, 128, L.W4_GRAPH | L.W4_A8)
        assert model.device_error() == 0
    finally:
        model.close()
    positions = np.arange(63, 128)
    worst, mism = compare_with_oracle(dims, lambda l: synth.layer_weights(dims, l), glob, lg, tk, 64, positions,
                                      cache_key="qwen7b-a8-64+64", act="int8")
    say(f"a8 full: max |logit err| {worst:.3e}; mismatches {mism} ({time.time() - t0:.0f}s)")
    assert worst <= LOGIT_ATOL
    assert not mism
