"""Prompt prefill on the GPU against the oracle: the W4A16 GEMM on matrix
cores, causal paged prefill attention, and the model's prefill call (logits,
greedy token, KV cache contents seen through the decode steps after it)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import int4_weight_only_dequant_amd as w4
from int4_weight_only_dequant_amd import _lib as L
from tests._tol import LOGIT_ATOL, assert_attn, assert_gemv, gemv_allclose_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 1.0 / np.sqrt(128.0)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


# ----------------------------------------------------------------- GEMM ----

@pytest.mark.parametrize("m,n,k", [(1, 64, 128), (64, 256, 128), (100, 320, 512), (77, 1000, 1024),
                                   (130, 3584, 3584), (512, 4608, 3584), (512, 3584, 18944),
                                   (512, 37888, 3584)])
def test_gemm_shapes(m, n, k):
    say(f"case: gemm M={m} N={n} K={k}")
    q, s, x = synth.gemm_case(m, n, k)
    pq, ps = w4.pack_int4_weights(q, s)
    y = w4.w4a16_gemm(_dev(pq), _dev(ps), _dev(x), n, k)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref = oracle.gemv(q, s, x)
    e = assert_gemv(y, ref, f"M={m} N={n} K={k}")
    say(f"  rel err {e:.3e} allclose {gemv_allclose_err(y, ref):.3f}")


def test_gemm_row_permutation_and_reuse():
    """Packed row order is kept (QKV permutation); a second call on the same
    workspace with a different shape is unaffected by the first."""
    m, n, k = 70, 384, 640
    q, s, x = synth.gemm_case(m, n, k, cfg=5)
    perm = np.random.default_rng(5).permutation(n).astype(np.int32)
    pq, ps = w4.pack_int4_weights(q, s, row_perm=perm)
    y1 = w4.w4a16_gemm(_dev(pq), _dev(ps), _dev(x), n, k)
    q2, s2, x2 = synth.gemm_case(512, 256, 2048, cfg=6)
    pq2, ps2 = w4.pack_int4_weights(q2, s2)
    y2 = w4.w4a16_gemm(_dev(pq2), _dev(ps2), _dev(x2), 256, 2048)
    torch.cuda.synchronize()
    assert_gemv(y1.cpu().numpy(), oracle.gemv(q[perm], s[perm], x), "permuted rows")
    assert_gemv(y2.cpu().numpy(), oracle.gemv(q2, s2, x2), "second shape")


def test_gemm_deterministic():
    q, s, x = synth.gemm_case(512, 3584, 3584, cfg=7)
    pq, ps = w4.pack_int4_weights(q, s)
    a = w4.w4a16_gemm(_dev(pq), _dev(ps), _dev(x), 3584, 3584).cpu().numpy()
    b = w4.w4a16_gemm(_dev(pq), _dev(ps), _dev(x), 3584, 3584).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------ attention ----

def _contiguous(pool, table, ctx):
    t = np.arange(ctx)
    return pool[table[t // 16], :, t % 16]          # [ctx, n_kvh, D]


def _gpu_attn(q, kp, vp, table, pos0):
    out = w4.paged_attn_prefill(_dev(q), _dev(kp), _dev(vp), _dev(table.astype(np.int32)), pos0, SCALE)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("pos0,m,n_qh,n_kvh", [(0, 1, 4, 1), (0, 45, 14, 2), (37, 100, 28, 4), (0, 512, 28, 4),
                                              (512, 96, 28, 4), (5, 33, 8, 8)])
def test_prefill_attention(pos0, m, n_qh, n_kvh):
    say(f"case: prefill attention pos0={pos0} M={m} heads {n_qh}/{n_kvh}")
    q, kp, vp, table = synth.prefill_attn_case(pos0, m, n_qh, n_kvh, n_pages=(pos0 + m + 15) // 16 + 3)
    got = _gpu_attn(q, kp, vp, table, pos0)
    ctx = pos0 + m
    K, V = _contiguous(kp, table, ctx), _contiguous(vp, table, ctx)
    Q = np.zeros((ctx, n_qh, 128), np.float16)
    Q[pos0:] = q
    ref = oracle.causal_attention(Q, K, V, SCALE)[pos0:]
    e = assert_attn(got, ref, f"pos0={pos0} M={m}")
    say(f"  max abs err {e:.3e}")


def test_prefill_attention_long_context_sampled():
    """A 512-token chunk after 7680 cached tokens (the long-context fill):
    sampled query rows against the oracle's paged attention."""
    pos0, m = 7680, 512
    say(f"case: prefill attention pos0={pos0} M={m}, sampled rows")
    q, kp, vp, table = synth.prefill_attn_case(pos0, m, 28, 4, n_pages=520, cfg=8)
    got = _gpu_attn(q, kp, vp, table, pos0)
    for r in (0, 1, 255, 300, 511):
        ref = oracle.paged_attention(q[r], kp, vp, table, pos0 + r + 1, SCALE)
        assert_attn(got[r], ref, f"row {r}")
    assert np.all(np.isfinite(got))


# ---------------------------------------------------------------- model ----

def _tiny(cfg, max_pages):
    dims = synth.TINY
    layers = [synth.layer_weights(dims, l, cfg=cfg) for l in range(dims.n_layers)]
    glob = synth.global_weights(dims, cfg=cfg)
    free = synth.page_free_list(max_pages, cfg=cfg)
    return dims, layers, glob, free


def _run(model, prompt, chunks, n_steps):
    """Prefill the prompt in the given chunk sizes, then n_steps greedy decode
    steps; returns logits [1 + n_steps, V] (after the prefill, then per step)
    and the token history."""
    model.reset(prompt)
    for c in chunks:
        model.prefill(c)
    out = [model.logits.clone()]
    for _ in range(n_steps):
        model.step()
        out.append(model.logits.clone())
    torch.cuda.synchronize()
    n = len(prompt) + n_steps + 1
    return torch.stack(out).cpu().numpy(), model.tokens[:n].cpu().numpy()


@pytest.mark.parametrize("n_prompt,chunks", [(40, [40]), (33, [16, 17]), (48, [20, 28]), (1, [1])])
def test_tiny_prefill_then_decode(n_prompt, chunks):
    dims, layers, glob, free = _tiny(104, 8)
    prompt = synth.prompt_ids(dims, n_prompt, cfg=104)
    n_steps = 24
    say(f"case: tiny model prefill {chunks} of a {n_prompt}-token prompt + {n_steps} steps")
    model = w4.DecodeModel(dims, lambda l: layers[l], glob, free, 8)
    try:
        lg, tk = _run(model, prompt, chunks, n_steps)
        assert model.device_error() == 0
        pt = model.page_table.cpu().numpy()
        n_used = (n_prompt + n_steps + 15) // 16
        assert np.array_equal(pt[:n_used], free[:n_used]) and np.all(pt[n_used:] == -1)
        assert model.pos == n_prompt + n_steps
        # the decode-only path on the same model gives the same tokens
        model.reset(prompt)
        for _ in range(n_prompt + n_steps):
            model.step()
        torch.cuda.synchronize()
        tk_dec = model.tokens[: n_prompt + n_steps + 1].cpu().numpy()
    finally:
        model.close()
    assert np.array_equal(tk[:n_prompt], prompt)
    assert np.array_equal(tk, tk_dec)
    positions = np.arange(n_prompt - 1, n_prompt + n_steps)
    ref = oracle.forward_teacher_forced(dims, layers, glob, tk[: positions[-1] + 1], positions)
    err = float(np.max(np.abs(lg - ref)))
    want = [oracle.argmax_first(r) for r in ref]
    say(f"  max |logit err| {err:.3e}")
    assert err <= LOGIT_ATOL
    assert list(tk[n_prompt:]) == want


@pytest.mark.parametrize("flags", [L.W4_MULTI | L.W4_GRAPH, L.W4_MULTI | L.W4_EAGER, L.W4_EAGER])
def test_tiny_prefill_then_other_step_variants(flags):
    """After a prefill call, the kernel-per-op step (graph and eager) and the
    eager persistent step continue the sequence with the same greedy tokens as
    the persistent graph, and logits within the two implementations' spread."""
    dims, layers, glob, free = _tiny(106, 8)
    n_prompt, n_steps = 40, 24
    prompt = synth.prompt_ids(dims, n_prompt, cfg=106)
    say(f"case: tiny model prefill {n_prompt} + {n_steps} steps with flags {flags}")
    model = w4.DecodeModel(dims, lambda l: layers[l], glob, free, 8)
    try:
        lg_ref, tk_ref = _run(model, prompt, [n_prompt], n_steps)
        model.reset(prompt)
        model.prefill(n_prompt)
        out = [model.logits.clone()]
        for _ in range(n_steps):
            model.step(flags)
            out.append(model.logits.clone())
        torch.cuda.synchronize()
        assert model.device_error() == 0
        lg = torch.stack(out).cpu().numpy()
        tk = model.tokens[: n_prompt + n_steps + 1].cpu().numpy()
        pt = model.page_table.cpu().numpy()
    finally:
        model.close()
    n_used = (n_prompt + n_steps + 15) // 16
    assert np.array_equal(pt[:n_used], free[:n_used]) and np.all(pt[n_used:] == -1)
    assert np.array_equal(tk, tk_ref)
    diff = float(np.max(np.abs(lg - lg_ref)))
    say(f"  max |logit diff| vs persistent graph {diff:.3e}")
    if flags & L.W4_MULTI:
        assert diff <= 1e-2
    else:
        assert diff == 0.0                     # eager launches of the same kernel: bitwise


def test_tiny_prefill_errors():
    dims, layers, glob, free = _tiny(105, 4)
    prompt = synth.prompt_ids(dims, 60, cfg=105)
    model = w4.DecodeModel(dims, lambda l: layers[l], glob, free, 4)
    try:
        model.reset(prompt)
        with pytest.raises(w4.W4Error) as e:
            w4.prefill(model, 3, 8)                 # out of sequence
        assert e.value.status == L.W4_ESTATE
        with pytest.raises(w4.W4Error) as e:
            model.prefill(0)
        assert e.value.status == L.W4_EINVAL
        with pytest.raises(w4.W4Error) as e:
            model.prefill(513)
        assert e.value.status == L.W4_EINVAL
        with pytest.raises(w4.W4Error) as e:
            model.prefill(65)                       # beyond 4 pages
        assert e.value.status == L.W4_ENOSPC
        model.prefill(60)
        for _ in range(4):
            model.step()
        with pytest.raises(w4.W4Error) as e:
            model.step()                            # position 64: pool full
        assert e.value.status == L.W4_ENOSPC
        assert model.device_error() == 0
    finally:
        model.close()


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_tiny_long_context_chunked_prefill_then_decode():
    """The long-context protocol on the small model: an 8192-token prompt
    filled by 16 chunked 512-token prefills over 520 shuffled pages, then
    greedy decode steps at positions 8192..; logits vs the oracle's
    teacher-forced pass over the whole sequence."""
    dims, layers, glob, free = _tiny(106, 520)
    n_prompt, n_steps = 8192, 16
    prompt = synth.prompt_ids(dims, n_prompt, cfg=106)
    say(f"case: tiny model, {n_prompt}-token prompt in 16 prefill chunks + {n_steps} steps, 520 pages")
    model = w4.DecodeModel(dims, lambda l: layers[l], glob, free, 520)
    try:
        lg, tk = _run(model, prompt, [512] * 16, n_steps)
        assert model.device_error() == 0
        pt = model.page_table.cpu().numpy()
    finally:
        model.close()
    n_used = (n_prompt + n_steps + 15) // 16
    assert np.array_equal(pt[:n_used], free[:n_used])
    positions = np.arange(n_prompt - 1, n_prompt + n_steps)
    ref = oracle.forward_teacher_forced(dims, layers, glob, tk[: positions[-1] + 1], positions)
    err = float(np.max(np.abs(lg - ref)))
    want = [oracle.argmax_first(r) for r in ref]
    say(f"  max |logit err| {err:.3e}")
    assert err <= LOGIT_ATOL
    assert list(tk[n_prompt:]) == want
