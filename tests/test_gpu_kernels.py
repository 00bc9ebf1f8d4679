"""Parity of the HIP kernels (called through the C ABI) with the CPU oracle."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import int4_weight_only_dequant_amd as w4
from int4_weight_only_dequant_amd import _lib as L
from tests._tol import assert_attn, assert_gemv, gemv_allclose_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a).to(DEV)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


WS_MARK = 0x57344731   # the streaming GEMV's workspace mark (first word)


def assert_ws_clean(ws):
    """After calls: the mark set, everything after the 256-byte header zero."""
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == WS_MARK, "workspace mark not set"
    assert int(torch.count_nonzero(ws[256:])) == 0, "workspace not left zero"


def _gpu_gemv(q, s, x):
    n, k = q.shape
    pq, ps = w4.pack_int4_weights(q, s)
    y = w4.w4a16_gemv(_dev(pq), _dev(ps), _dev(x), n, k)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ----------------------------------------------------------------- GEMV ----

def test_gemv_cfg0():
    say("case: gemv cfg0 3584x3584 seed 0")
    q, s, x = synth.gemv_cfg0()
    y = _gpu_gemv(q, s, x)
    ref = oracle.gemv(q, s, x)
    e = assert_gemv(y, ref, "cfg0")
    say(f"cfg0 rel err {e:.3e} allclose {gemv_allclose_err(y, ref):.3f}")


@pytest.mark.parametrize("n,k", [(1, 128), (64, 128), (100, 384), (257, 3584), (4608, 3584),
                                 (3584, 18944), (37888, 3584), (130, 1024)])
def test_gemv_shapes(n, k):
    say(f"case: gemv N={n} K={k}")
    q, s, x = synth.gemv_case(n, k, cfg=94)
    y = _gpu_gemv(q, s, x)
    assert_gemv(y, oracle.gemv(q, s, x), f"N={n} K={k}")


def test_gemv_edge_values():
    """Extreme codes, tiny/huge scales and fp16-subnormal activations."""
    say("case: gemv edge values")
    n, k = 128, 512
    r = np.random.default_rng(3)
    q = np.where(r.random((n, k)) < 0.5, -8, 7).astype(np.int8)
    s = np.full((n, k // 128), 1.0, np.float16)
    s[:, 0] = np.float16(6e-8)          # subnormal scale
    s[:, 1] = np.float16(60000.0)
    s[:, 2] = np.float16(-2.0)
    x = (r.standard_normal(k) * 1e-3).astype(np.float16)
    x[::7] = np.float16(3e-7)           # fp16 subnormals
    x[1::11] = 0
    y = _gpu_gemv(q, s, x)
    assert_gemv(y, oracle.gemv(q, s, x), "edge")


def test_gemv_deterministic_and_ws_reuse():
    say("case: gemv repeat determinism")
    q, s, x = synth.gemv_case(3584, 18944, cfg=95)
    pq, ps = w4.pack_int4_weights(q, s)
    dq, ds, dx = _dev(pq), _dev(ps), _dev(x)
    first = w4.w4a16_gemv(dq, ds, dx, 3584, 18944).clone()
    for _ in range(50):
        y = w4.w4a16_gemv(dq, ds, dx, 3584, 18944)
    torch.cuda.synchronize()
    assert torch.equal(first, y)


def test_gemv_shared_workspace_across_shapes_left_zero():
    """One caller-owned workspace, zeroed once, serves GEMVs of different
    shapes back to back: each result equals the oracle's and the bitwise
    result of a fresh workspace, and the workspace is all zero after every
    call (the contract that lets calls skip clearing it)."""
    lib = L.lib()
    shapes = [(3584, 18944), (37888, 3584), (100, 384), (3584, 3584), (257, 3584)]
    need = max(lib.w4_gemv_ws_bytes(n, k) for n, k in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    for i, (n, k) in enumerate(shapes):
        say(f"case: shared workspace, call {i}: N={n} K={k}")
        q, s, x = synth.gemv_case(n, k, cfg=97 + i)
        pq, ps = w4.pack_int4_weights(q, s)
        dq, ds, dx = _dev(pq), _dev(ps), _dev(x)
        y = torch.empty(n, dtype=torch.float16, device=DEV)
        L.check(lib.w4a16_gemv(dq.data_ptr(), ds.data_ptr(), dx.data_ptr(), y.data_ptr(), n, k,
                               ws.data_ptr(), ws.numel(), st))
        torch.cuda.synchronize()
        assert_ws_clean(ws)
        fresh = w4.w4a16_gemv(dq, ds, dx, n, k).clone()
        torch.cuda.synchronize()
        assert torch.equal(y, fresh)
        assert_gemv(y.cpu().numpy(), oracle.gemv(q, s, x), f"shared ws N={n} K={k}")


# ------------------------------------------------------------------ MLP ----

def test_gemv_workspace_never_zeroed_gives_nan():
    """Memory that was never zeroed (its first word neither 0 nor the mark)
    is refused visibly: y is all NaN and the workspace is left as it was;
    once zeroed, the same call is correct."""
    n, k = 3584, 3584
    say(f"case: gemv N={n} K={k} on a workspace of 0xAB bytes")
    q, s, x = synth.gemv_case(n, k, cfg=95)
    pq, ps = w4.pack_int4_weights(q, s)
    dq, ds, dx = _dev(pq), _dev(ps), _dev(x)
    lib = L.lib()
    ws = torch.full((lib.w4_gemv_ws_bytes(n, k),), 0xAB, dtype=torch.uint8, device=DEV)
    y = torch.empty(n, dtype=torch.float16, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    L.check(lib.w4a16_gemv(dq.data_ptr(), ds.data_ptr(), dx.data_ptr(), y.data_ptr(), n, k, ws.data_ptr(),
                           ws.numel(), st))
    torch.cuda.synchronize()
    assert bool(torch.isnan(y.float()).all()), "a never-zeroed workspace must give NaN outputs"
    assert bool((ws == 0xAB).all()), "a refused workspace is left untouched"
    ws.zero_()
    L.check(lib.w4a16_gemv(dq.data_ptr(), ds.data_ptr(), dx.data_ptr(), y.data_ptr(), n, k, ws.data_ptr(),
                           ws.numel(), st))
    torch.cuda.synchronize()
    assert_gemv(y.cpu().numpy(), oracle.gemv(q, s, x), "after zeroing")
    assert_ws_clean(ws)


def test_mlp_cfg1():
    say("case: mlp cfg1 d=3584 f=18944")
    m = synth.mlp_cfg1()
    d, f = 3584, 18944
    cfg = L.ModelConfig(d_model=d, d_ff=f, n_layers=1, n_q_heads=28, n_kv_heads=4, head_dim=128,
                        vocab=1, max_pages=1, eps=1e-6, theta=1e6)
    perm = w4.model_row_perm(L.W4_PERM_GATE_UP, cfg)
    gq = np.concatenate([m["gate"][0], m["up"][0]])
    gs = np.concatenate([m["gate"][1], m["up"][1]])
    pgq, pgs = w4.pack_int4_weights(gq, gs, row_perm=perm)
    pdq, pds = w4.pack_int4_weights(*m["down"])
    h, y = w4.w4a16_mlp(_dev(pgq), _dev(pgs), _dev(pdq), _dev(pds), _dev(m["x"]), d, f)
    torch.cuda.synchronize()
    h = h.cpu().numpy()
    y = y.cpu().numpy()
    # h against the oracle's SwiGLU of the oracle GEMVs (fp16 storage point on both sides)
    g_ref = oracle.gemv(*m["gate"], m["x"])
    u_ref = oracle.gemv(*m["up"], m["x"])
    h_ref = oracle.swiglu(g_ref, u_ref)
    assert_gemv(h, h_ref, "swiglu h")
    # down on the GPU's own h (the intermediate tolerance reading)
    assert_gemv(y, oracle.gemv(*m["down"], h), "down")
    # end to end against the oracle's own h
    _, y_ref = oracle.mlp(m["x"], m["gate"], m["up"], m["down"])
    say(f"mlp end-to-end rel err {np.max(np.abs(y - y_ref) / np.maximum(np.abs(y_ref), 1e-3)):.3e}")


def _mlp_operands(d, f, seed_cfg):
    m = synth.mlp_cfg1(seed=seed_cfg, d=d, f=f)
    cfg = L.ModelConfig(d_model=d, d_ff=f, n_layers=1, n_q_heads=max(1, d // 128), n_kv_heads=1, head_dim=128,
                        vocab=1, max_pages=1, eps=1e-6, theta=1e6)
    perm = w4.model_row_perm(L.W4_PERM_GATE_UP, cfg)
    pgq, pgs = w4.pack_int4_weights(np.concatenate([m["gate"][0], m["up"][0]]),
                                    np.concatenate([m["gate"][1], m["up"][1]]), row_perm=perm)
    pdq, pds = w4.pack_int4_weights(*m["down"])
    return m, [_dev(a) for a in (pgq, pgs, pdq, pds, m["x"])]


def _mlp_raw(ops, d, f, ws):
    """One w4a16_mlp call through the C ABI on a caller-held workspace."""
    lib = L.lib()
    h = torch.empty(f, dtype=torch.float16, device=DEV)
    y = torch.empty(d, dtype=torch.float16, device=DEV)
    L.check(lib.w4a16_mlp(*[t.data_ptr() for t in ops], h.data_ptr(), y.data_ptr(), d, f, ws.data_ptr(),
                          ws.numel(), torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return h.cpu().numpy(), y.cpu().numpy()


@pytest.mark.parametrize("d,f", [(128, 128), (256, 384), (384, 1280), (1024, 2816), (3584, 18944)])
def test_mlp_shapes_and_workspace_reuse(d, f):
    """Small, ragged and full shapes; five calls on one workspace give the
    same bits as the first, and the workspace is left zero."""
    say(f"case: mlp D={d} F={f}, 5 calls on one workspace")
    m, ops = _mlp_operands(d, f, 131)
    ws = torch.zeros(max(L.lib().w4_mlp_ws_bytes(d, f), 256), dtype=torch.uint8, device=DEV)
    h0, y0 = _mlp_raw(ops, d, f, ws)
    g_ref = oracle.gemv(*m["gate"], m["x"])
    u_ref = oracle.gemv(*m["up"], m["x"])
    assert_gemv(h0, oracle.swiglu(g_ref, u_ref), f"h D={d} F={f}")
    assert_gemv(y0, oracle.gemv(*m["down"], h0), f"y D={d} F={f}")
    for i in range(4):
        h, y = _mlp_raw(ops, d, f, ws)
        assert np.array_equal(h.view(np.uint16), h0.view(np.uint16)), f"call {i + 2}: h differs"
        assert np.array_equal(y.view(np.uint16), y0.view(np.uint16)), f"call {i + 2}: y differs"
    assert_ws_clean(ws)


# ------------------------------------------------------------ attention ----

def _gpu_attn(q, kp, vp, table, ctx, n_pages_max=None, scale=1 / math.sqrt(128)):
    if n_pages_max is not None and n_pages_max > len(table):
        table = np.concatenate([table, np.zeros(n_pages_max - len(table), np.int32)])
    out = w4.paged_attn_decode(_dev(q), _dev(kp), _dev(vp), _dev(table.astype(np.int32)), ctx, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_attn_cfg2():
    say("case: attention cfg2 ctx 640, 40 shuffled pages")
    q, kp, vp, table = synth.attn_cfg2()
    o = _gpu_attn(q, kp, vp, table, 640)
    ref = oracle.paged_attention(q, kp, vp, table, 640, 1 / math.sqrt(128))
    say(f"cfg2 abs err {assert_attn(o, ref, 'cfg2'):.3e}")


@pytest.mark.parametrize("ctx", [1, 2, 15, 16, 17, 31, 33, 100, 639, 640])
def test_attn_ctx_sweep(ctx):
    say(f"case: attention ctx {ctx} (pool 40 pages)")
    q, kp, vp, table = synth.attn_case(640, cfg=96)
    o = _gpu_attn(q, kp, vp, table, ctx)
    ref = oracle.paged_attention(q, kp, vp, table, ctx, 1 / math.sqrt(128))
    assert_attn(o, ref, f"ctx={ctx}")


def test_attn_long_context_8193():
    say("case: attention ctx 8193, 520-page pool")
    q, kp, vp, table = synth.attn_case(8193, n_pages=520, cfg=97)
    o = _gpu_attn(q, kp, vp, table, 8193, n_pages_max=520)
    ref = oracle.paged_attention(q, kp, vp, table, 8193, 1 / math.sqrt(128))
    assert_attn(o, ref, "ctx=8193")


@pytest.mark.parametrize("n_pages,ctx", [(1, 5), (1, 16), (2, 17), (3, 40), (128, 2041), (512, 8192),
                                         (2048, 32763)])
def test_attn_split_geometry(n_pages, ctx):
    """Pools from 1 to 2048 pages: one split per kv head up to 64 splits of
    32 pages, so the last-arriver merge runs from one partial to two full
    rounds of 32; ragged and full last pages."""
    say(f"case: attention ctx {ctx}, {n_pages}-page pool")
    q, kp, vp, table = synth.attn_case(ctx, n_pages=n_pages, cfg=107)
    o = _gpu_attn(q, kp, vp, table, ctx, n_pages_max=n_pages)
    ref = oracle.paged_attention(q, kp, vp, table, ctx, 1 / math.sqrt(128))
    say(f"  abs err {assert_attn(o, ref, f'ctx={ctx} pool={n_pages}'):.3e}")


def test_attn_long_context_repeat_bit_identical():
    """64 splits per kv head (two merge rounds): 200 calls give bit-identical outputs."""
    say("case: attention ctx 8190 x200 repeat, 512-page pool")
    q, kp, vp, table = synth.attn_case(8190, n_pages=512, cfg=108)
    dq, dk, dv, dt = _dev(q), _dev(kp), _dev(vp), _dev(table)
    first = w4.paged_attn_decode(dq, dk, dv, dt, 8190, 1 / math.sqrt(128)).clone()
    outs = [w4.paged_attn_decode(dq, dk, dv, dt, 8190, 1 / math.sqrt(128)).clone() for _ in range(200)]
    torch.cuda.synchronize()
    assert all(torch.equal(first, o) for o in outs)


def test_attn_alternating_inputs_on_one_workspace():
    """The split partials are re-read with plain loads by the last work-group:
    calls alternating two different queries (and contexts) on one workspace
    must each reproduce their own first output bit for bit, so no call reads
    a partial left in a cache by the call before."""
    say("case: attention alternating inputs x100, 512-page pool")
    q, kp, vp, table = synth.attn_case(8190, n_pages=512, cfg=109)
    q2 = synth.attn_case(8190, n_pages=512, cfg=110)[0]
    dq, dq2, dk, dv, dt = _dev(q), _dev(q2), _dev(kp), _dev(vp), _dev(table)
    scale = 1 / math.sqrt(128)
    a0 = w4.paged_attn_decode(dq, dk, dv, dt, 8190, scale).clone()
    b0 = w4.paged_attn_decode(dq2, dk, dv, dt, 7001, scale).clone()
    outs = []
    for _ in range(100):
        outs.append((w4.paged_attn_decode(dq, dk, dv, dt, 8190, scale).clone(),
                     w4.paged_attn_decode(dq2, dk, dv, dt, 7001, scale).clone()))
    torch.cuda.synchronize()
    assert all(torch.equal(a, a0) and torch.equal(b, b0) for a, b in outs)
    ref = oracle.paged_attention(q2, kp, vp, table, 7001, scale)
    assert_attn(b0.cpu().numpy(), ref, "ctx=7001")


def test_attn_one_token_is_v_row():
    say("case: attention one token")
    q, kp, vp, table = synth.attn_case(640, cfg=98)
    o = _gpu_attn(q, kp, vp, table, 1)
    want = np.stack([vp[table[0], h // 7, 0] for h in range(28)])
    assert np.array_equal(o.view(np.uint16), want.view(np.uint16))


def test_attn_shuffled_equals_contiguous_bitwise():
    say("case: attention shuffled vs contiguous")
    q, kp, vp, table = synth.attn_case(600, cfg=99)
    kc, vc = kp[table], vp[table]
    o1 = _gpu_attn(q, kp, vp, table, 600)
    o2 = _gpu_attn(q, kc, vc, np.arange(len(table), dtype=np.int32), 600)
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))


def test_attn_gqa_and_scale_variants():
    for n_qh, n_kvh in [(28, 4), (8, 4), (16, 4), (8, 1), (32, 4), (4, 4), (8, 8)]:
        say(f"case: attention GQA {n_qh}/{n_kvh}")
        q, kp, vp, table = synth.attn_case(77, n_qh=n_qh, n_kvh=n_kvh, n_pages=6, cfg=100)
        o = _gpu_attn(q, kp, vp, table, 77, scale=0.05)
        ref = oracle.paged_attention(q, kp, vp, table, 77, 0.05)
        assert_attn(o, ref, f"gqa {n_qh}/{n_kvh}")


@pytest.mark.parametrize("scale", [1.0, 4.0])
def test_attn_peaked_softmax(scale):
    """Scores spread over tens of units (base-2 exponents past -100): most
    weights underflow, one or a few tokens carry the output; the weights' fp16
    hi + lo pair and the split merge must still match the oracle."""
    say(f"case: attention ctx 1000, scale {scale}")
    q, kp, vp, table = synth.attn_case(1000, n_pages=70, cfg=111)
    o = _gpu_attn(q, kp, vp, table, 1000, scale=scale, n_pages_max=70)
    ref = oracle.paged_attention(q, kp, vp, table, 1000, scale)
    say(f"  abs err {assert_attn(o, ref, f'scale={scale}'):.3e}")


def test_attn_repeat_bit_identical():
    """Race detector: 1000 calls must give bit-identical outputs (tail page included)."""
    say("case: attention x1000 repeat")
    q, kp, vp, table = synth.attn_case(637, cfg=101)
    dq, dk, dv, dt = _dev(q), _dev(kp), _dev(vp), _dev(table)
    first = w4.paged_attn_decode(dq, dk, dv, dt, 637, 1 / math.sqrt(128)).clone()
    outs = [w4.paged_attn_decode(dq, dk, dv, dt, 637, 1 / math.sqrt(128)).clone() for _ in range(1000)]
    torch.cuda.synchronize()
    assert all(torch.equal(first, o) for o in outs)
