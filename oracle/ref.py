"""Plain, slow, float64 reference for the W4A16 batch-1 decode step.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests, the smoke
check and the CPU-baseline timing, never by the product path.

Sources (web pages on the "annotated-llm-runtime" project):

* [TS] "Building a Custom LLM Inference Runtime for Qwen2.5-Coder-7B on NVIDIA
  H100 Hopper Architecture" (techsurvey.info);
* [SP] "The Architecture of Modern Inference: A Deep Dive into the Development
  of the Annotated LLM Runtime for NVIDIA Hopper GPUs" (snapost.net);
* [AI] "How To Build Your Own LLM Runtime From Scratch" (aissential.tech).

The pages fix: symmetric group-wise int4 projection weights, group 128, one
fp16 scale per group, fp16 embeddings / norms / lm_head ([TS] "Technical
Specifications and Hardware Alignment"); fp16 activations into the quantised
GEMV ([TS] "Engineering Challenges", item 3); a paged KV cache of 16-token
pages ([TS] "Technical Specifications…"; [AI] "Method"); attention as softmax
plus weighted-V accumulation ([SP] "Three Critical Engineering Challenges",
item 1).  Everything else (RoPE pairing, GQA grouping, QKV bias, norm form,
SwiGLU ordering, argmax tie-break, fp16 storage points) is a stated reading of
the Qwen2.5-7B decode workload, listed with the design notes.

fp16 storage points (round to nearest even): the GEMV inputs a, o, h, a2, xf;
q, k, v after RoPE; the K/V cache.  Everything else stays float64.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64

__all__ = [
    "f16", "deq", "gemv", "quantize_int4", "quantize_act_int8", "act_int8", "gemv_w4a8", "rmsnorm", "rope", "silu", "swiglu", "softmax",
    "paged_attention", "causal_attention", "mlp", "argmax_first",
    "KVCache", "layer_step", "decode_step", "forward_teacher_forced",
]


def f16(x) -> np.ndarray:
    """Round to IEEE binary16 (numpy converts float64 -> float16 directly, RNE)."""
    return np.asarray(x, dtype=F64).astype(np.float16)


# --------------------------------------------------------------------------
# W4A16 GEMV  ([TS] "Technical Specifications and Hardware Alignment")
# --------------------------------------------------------------------------

def deq(q: np.ndarray, s: np.ndarray, group: int = 128) -> np.ndarray:
    """Dequantised weights W[n, k] = q[n, k] * s[n, k // group], in float64.

    Symmetric (no zero point): the 4-bit code times its group's fp16 scale.
    """
    q = np.asarray(q)
    s = np.asarray(s)
    n, k = q.shape
    if k % group or s.shape != (n, k // group):
        raise ValueError(f"codes {q.shape} and scales {s.shape} do not match group {group}")
    per_element_scale = np.repeat(s.astype(F64), group, axis=1)
    return q.astype(F64) * per_element_scale


def gemv(q: np.ndarray, s: np.ndarray, x: np.ndarray, group: int = 128) -> np.ndarray:
    """y = deq(q, s) @ x in float64 (x may be a vector [K] or rows [T, K] -> [T, N])."""
    w = deq(q, s, group)
    x = np.asarray(x, dtype=F64)
    if x.ndim == 1:
        return w @ x
    return x @ w.T


# --------------------------------------------------------------------------
# fp16 -> int4 weight quantiser (the step before the packed weights: the
# pages store symmetric group-wise INT4 weights with one fp16 scale per group
# of 128, [TS] "Technical Specifications and Hardware Alignment" and
# ".nanoqwen File Format"; they do not give the quantiser).  Reading: per
# group, scale = fp16(max|w| / 7) (the exact quotient rounded once to fp16),
# code = clamp(round-half-even(w / scale), -8, 7); a group whose scale
# rounds to zero gets zero codes.
# --------------------------------------------------------------------------

def quantize_int4(w: np.ndarray, group: int = 128) -> tuple:
    """(codes int8 [N, K] in [-8, 7], scales fp16 [N, K / group]) of fp16 weights."""
    w = np.asarray(w, dtype=np.float16)
    n, k = w.shape
    if k % group:
        raise ValueError(f"K={k} is not a multiple of {group}")
    wg = w.astype(F64).reshape(n, k // group, group)
    amax = np.max(np.abs(wg), axis=2)
    scales = (amax / 7.0).astype(np.float16)              # fp64 quotient, one rounding to fp16
    s64 = scales.astype(F64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s64 > 0, np.rint(wg / np.where(s64 > 0, s64, 1.0)), 0.0)
    codes = np.clip(r, -8, 7).astype(np.int8).reshape(n, k)
    return codes, scales


# --------------------------------------------------------------------------
# W4A8 GEMV: int8 activations ("Path A" of [TS] "Engineering Challenges",
# item 3, and [SP] "Three Critical Engineering Challenges", item 3: weights and
# activations both integer, so the inner products run on integer dot-product
# instructions, after a separate step that quantises the fp16 activations).
# The pages do not give the activation quantiser; the reading used here is
# symmetric, per group of 128 along K (the weights' groups): one float32
# scale per group, s = max|x| / 127 rounded to float32, codes
# round-half-even(x / s) in float32, clamped to [-127, 127]; an all-zero group
# has scale 0 and zero codes.
# --------------------------------------------------------------------------

def quantize_act_int8(x: np.ndarray, group: int = 128) -> tuple:
    """(codes int8 [K], scales float32 [K / group]) of an fp16 activation vector."""
    x = np.asarray(x, dtype=np.float16)
    k = x.shape[0]
    if k % group:
        raise ValueError(f"K={k} is not a multiple of {group}")
    xg = x.astype(np.float32).reshape(k // group, group)
    amax = np.max(np.abs(xg), axis=1)
    scales = (amax / np.float32(127.0)).astype(np.float32)
    codes = np.zeros_like(xg, dtype=np.int8)
    for g in range(k // group):
        if scales[g] == 0:
            continue
        r = np.rint(xg[g] / scales[g]).astype(np.float32)     # float32 quotient, ties to even
        codes[g] = np.clip(r, -127, 127).astype(np.int8)
    return codes.reshape(k), scales


def act_int8(x: np.ndarray, group: int = 128) -> np.ndarray:
    """What an int8-activation GEMV multiplies: the fp16 input x (a vector [K]
    or rows [T, K]) quantised per group as quantize_act_int8 does, returned
    dequantised (codes times scale) in float64.  gemv(q, s, act_int8(x)) is
    gemv_w4a8 of the quantised x.  Rows are quantised independently; the
    arithmetic is quantize_act_int8's (float32 scale and quotient, ties to
    even, clamp), written over all groups at once."""
    x = np.asarray(x, dtype=np.float16)
    lead, k = x.shape[:-1], x.shape[-1]
    if k % group:
        raise ValueError(f"K={k} is not a multiple of {group}")
    xg = x.astype(np.float32).reshape(*lead, k // group, group)
    scales = (np.max(np.abs(xg), axis=-1) / np.float32(127.0)).astype(np.float32)
    nz = scales != 0
    safe = np.where(nz, scales, np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.rint(xg / safe[..., None]).astype(np.float32), -127, 127)
    codes = np.where(nz[..., None], codes, np.float32(0.0))
    return (codes.astype(F64) * scales[..., None].astype(F64)).reshape(*lead, k)


def gemv_w4a8(q: np.ndarray, s: np.ndarray, xq: np.ndarray, xs: np.ndarray, group: int = 128) -> np.ndarray:
    """y = deq(q, s) @ (xq * xs per group), in float64: the plain definition of
    the integer-activation GEMV (every product q * s * xq * xs is exact in fp64)."""
    xdeq = np.asarray(xq, dtype=F64) * np.repeat(np.asarray(xs, dtype=F64), group)
    return deq(q, s, group) @ xdeq


# --------------------------------------------------------------------------
# glue: RMSNorm, RoPE, SwiGLU
# --------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis, float64 (no rounding)."""
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=F64)


def rope(z: np.ndarray, pos, theta: float = 1e6) -> np.ndarray:
    """Rotary embedding with half-split pairs (i, i + D/2).

    z: [..., heads, D] (or [heads, D] for one position).  pos: a scalar or an
    array whose shape matches z's leading axes.  Pair i turns by the angle
    pos * theta ** (-2 i / D).
    """
    z = np.asarray(z, dtype=F64)
    d = z.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=F64)
    inv_freq = theta ** (-2.0 * i / d)
    p = np.asarray(pos, dtype=F64)
    phi = p[..., None] * inv_freq                 # [..., half]
    phi = phi[..., None, :]                       # broadcast over heads
    c, s = np.cos(phi), np.sin(phi)
    lo, hi = z[..., :half], z[..., half:]
    return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=F64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """silu(gate) * up (float64; the caller rounds to fp16)."""
    return silu(g) * np.asarray(u, dtype=F64)


def softmax(scores: np.ndarray) -> np.ndarray:
    """Numerically stable softmax over the last axis, float64."""
    s = np.asarray(scores, dtype=F64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def mlp(x: np.ndarray, gate, up, down) -> tuple:
    """The MLP decode block on one token: h = fp16(silu(Wg x) * (Wu x)), y = Wd h.

    Returns (h fp16, y float64).
    """
    g = gemv(*gate, x)
    u = gemv(*up, x)
    h = f16(swiglu(g, u))
    return h, gemv(*down, h)


# --------------------------------------------------------------------------
# attention  ([TS] "Engineering Challenges" item 1; [AI] "Method")
# --------------------------------------------------------------------------

def paged_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                    page_table: np.ndarray, ctx: int, scale: float,
                    page: int = 16) -> np.ndarray:
    """Decode attention of one query token over ctx cached tokens, float64.

    q [n_qh, D]; pools [n_phys, n_kvh, page, D] in physical page order; token t
    lives in physical page page_table[t // page], slot t % page.  Query head h
    reads kv head h // (n_qh / n_kvh).  Softmax over all ctx scores, then the
    weighted sum of the V rows.
    """
    q = np.asarray(q, dtype=F64)
    n_qh, d = q.shape
    n_kvh = k_pool.shape[1]
    if n_qh % n_kvh:
        raise ValueError("query heads must be a multiple of kv heads")
    grp = n_qh // n_kvh
    if ctx < 1:
        raise ValueError("context must hold at least one token")
    out = np.empty((n_qh, d), dtype=F64)
    for j in range(n_kvh):
        keys = np.empty((ctx, d), dtype=F64)
        vals = np.empty((ctx, d), dtype=F64)
        for t in range(ctx):
            phys = int(page_table[t // page])
            keys[t] = k_pool[phys, j, t % page]
            vals[t] = v_pool[phys, j, t % page]
        for h in range(j * grp, (j + 1) * grp):
            scores = (keys @ q[h]) * scale
            w = softmax(scores)
            out[h] = w @ vals
    return out


def causal_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Teacher-forced attention over a contiguous cache: position p sees 0..p.

    Q [T, n_qh, D], K and V [T, n_kvh, D] -> [T, n_qh, D], float64.
    """
    T, n_qh, d = Q.shape
    n_kvh = K.shape[1]
    grp = n_qh // n_kvh
    out = np.empty((T, n_qh, d), dtype=F64)
    Kf = K.astype(F64)
    Vf = V.astype(F64)
    Qf = Q.astype(F64)
    for p in range(T):
        for j in range(n_kvh):
            heads = slice(j * grp, (j + 1) * grp)
            scores = (Qf[p, heads] @ Kf[: p + 1, j].T) * scale   # [grp, p+1]
            out[p, heads] = softmax(scores) @ Vf[: p + 1, j]
    return out


def argmax_first(logits: np.ndarray) -> int:
    """Greedy choice: the lowest index among the maxima."""
    return int(np.argmax(np.asarray(logits)))


# --------------------------------------------------------------------------
# decoder: sequential decode step and batched teacher-forced pass
# --------------------------------------------------------------------------

class KVCache:
    """Per-layer paged K/V pools [n_pages, n_kvh, page, D] fp16 and one page table.

    page_table[i] is the physical page of logical page i; it is shared by all
    layers and given up front (the free-list order).
    """

    def __init__(self, dims, n_pages: int, page_table: np.ndarray):
        self.dims = dims
        shape = (n_pages, dims.n_kv_heads, dims.page, dims.head_dim)
        self.k = [np.zeros(shape, np.float16) for _ in range(dims.n_layers)]
        self.v = [np.zeros(shape, np.float16) for _ in range(dims.n_layers)]
        self.page_table = np.asarray(page_table, dtype=np.int32)

    def store(self, layer: int, pos: int, k: np.ndarray, v: np.ndarray) -> None:
        page = self.dims.page
        phys = int(self.page_table[pos // page])
        self.k[layer][phys, :, pos % page] = k
        self.v[layer][phys, :, pos % page] = v


def _split_qkv(dims, y):
    qd, kd = dims.q_dim, dims.kv_dim
    lead = y.shape[:-1]
    q = y[..., :qd].reshape(*lead, dims.n_q_heads, dims.head_dim)
    k = y[..., qd:qd + kd].reshape(*lead, dims.n_kv_heads, dims.head_dim)
    v = y[..., qd + kd:].reshape(*lead, dims.n_kv_heads, dims.head_dim)
    return q, k, v


def _gemv_input(act: str):
    """The four int4 GEMV inputs as the projections see them: the fp16 vector
    itself (act="f16"), or its per-group int8 quantisation (act="int8", the
    pages' integer-activation path, [TS] "Engineering Challenges" item 3)."""
    if act == "f16":
        return lambda v: v
    if act == "int8":
        return act_int8
    raise ValueError(f"unknown activation mode {act!r}")


def layer_step(dims, lw, x: np.ndarray, pos: int, cache: KVCache, layer: int,
               trace: dict | None = None, act: str = "f16") -> np.ndarray:
    """One decoder layer for the token at position pos; returns the new residual.

    x is the float64 residual [d].  The layer's own k, v are appended to the
    cache before attention, so the token attends to positions 0..pos.  act
    selects how the int4 GEMVs take their fp16 inputs (see _gemv_input).
    """
    inp = _gemv_input(act)
    a = f16(rmsnorm(x, lw.ln1, dims.eps))
    y = gemv(*lw.qkv, inp(a)) + lw.bqkv.astype(F64)
    q, k, v = _split_qkv(dims, y)
    q = f16(rope(q, pos, dims.theta))
    k = f16(rope(k, pos, dims.theta))
    v = f16(v)
    cache.store(layer, pos, k, v)
    o = paged_attention(q, cache.k[layer], cache.v[layer], cache.page_table,
                        pos + 1, 1.0 / np.sqrt(dims.head_dim), dims.page)
    o = f16(o).reshape(-1)
    x1 = x + gemv(*lw.o, inp(o))
    a2 = f16(rmsnorm(x1, lw.ln2, dims.eps))
    g, u = gemv(*lw.gate, inp(a2)), gemv(*lw.up, inp(a2))
    h = f16(swiglu(g, u))
    x2 = x1 + gemv(*lw.down, inp(h))
    if trace is not None:
        trace.update(a=a, qkv=y, q=q, k=k, v=v, o=o, x1=x1, a2=a2, g=g, u=u, h=h, x=x2)
    return x2


def decode_step(dims, layers, glob, cache: KVCache, token: int, pos: int, act: str = "f16") -> np.ndarray:
    """Logits (float64 [vocab]) for the token at position pos, updating the cache.

    ``layers`` is a sequence of LayerWeights or a callable layer -> LayerWeights.
    """
    get = layers if callable(layers) else layers.__getitem__
    x = glob.embed[int(token)].astype(F64)
    for layer in range(dims.n_layers):
        x = layer_step(dims, get(layer), x, pos, cache, layer, act=act)
    xf = f16(rmsnorm(x, glob.lnf, dims.eps))
    return glob.lm_head.astype(F64) @ xf.astype(F64)


def forward_teacher_forced(dims, layers, glob, tokens: np.ndarray, out_positions,
                           progress=None, act: str = "f16") -> np.ndarray:
    """Logits at out_positions for the token sequence, all positions in one pass.

    Position p holds tokens[p] and attends to 0..p.  Per position this is the
    same arithmetic as ``decode_step`` (contiguous cache instead of pages), so
    each weight matrix is dequantised once per layer.  Returns float64
    [len(out_positions), vocab].
    """
    get = layers if callable(layers) else layers.__getitem__
    inp = _gemv_input(act)
    tokens = np.asarray(tokens)
    T = len(tokens)
    pos = np.arange(T)
    X = glob.embed[tokens].astype(F64)
    scale = 1.0 / np.sqrt(dims.head_dim)
    for layer in range(dims.n_layers):
        lw = get(layer)
        A = f16(rmsnorm(X, lw.ln1, dims.eps))
        Y = gemv(*lw.qkv, inp(A)) + lw.bqkv.astype(F64)
        Q, K, V = _split_qkv(dims, Y)
        Q = f16(rope(Q, pos, dims.theta))
        K = f16(rope(K, pos, dims.theta))
        V = f16(V)
        O = f16(causal_attention(Q, K, V, scale)).reshape(T, -1)
        X = X + gemv(*lw.o, inp(O))
        A2 = f16(rmsnorm(X, lw.ln2, dims.eps))
        Hh = f16(swiglu(gemv(*lw.gate, inp(A2)), gemv(*lw.up, inp(A2))))
        X = X + gemv(*lw.down, inp(Hh))
        del lw
        if progress is not None:
            progress(layer)
    idx = np.asarray(out_positions)
    XF = f16(rmsnorm(X[idx], glob.lnf, dims.eps)).astype(F64)
    logits = np.empty((len(idx), dims.vocab), dtype=F64)
    step = 16384                                  # bounds the float64 copy of lm_head
    for r0 in range(0, dims.vocab, step):
        logits[:, r0:r0 + step] = XF @ glob.lm_head[r0:r0 + step].astype(F64).T
    return logits
