"""Seeded synthetic inputs for the W4A16 batch-1 decode step.

This module only draws random numbers and arranges them into arrays of the
shapes the workloads use.  It holds none of the method's arithmetic (no
dequantisation, no norms, no attention); both the CPU oracle and the HIP path
consume what it produces, so the two sides see identical inputs.

Every tensor has its own stream::

    numpy.random.default_rng(SeedSequence([seed, cfg, layer, tensor_id]))

with ``layer = 1000`` for tensors that do not belong to a decoder layer.
Tensor ids: 0/1 QKV codes/scales, 2/3 O, 4/5 gate, 6/7 up, 8/9 down,
10 pre-attention norm, 11 pre-MLP norm, 12 QKV bias, 20 embeddings,
21 lm_head, 22 final norm, 30 prompt ids, 31 page free list,
40 activation x, 41 attention q, 42 K pool, 43 V pool, 44 prefill
activation rows X, 45 prefill queries Q.

Distributions (the workloads' recipe):

* int4 codes: uniform integers in [-8, 7];
* group scales (one per 128 consecutive K elements of a row):
  fp16(|N(0,1)| * 0.02 + 1e-3);
* activations, q, K, V, embeddings: fp16 N(0,1);
* norm weights fp16(1 + 0.1 N(0,1)); QKV bias fp16(0.1 N(0,1));
  lm_head fp16(0.02 N(0,1));
* prompt ids uniform in [0, vocab); physical page order a random permutation.

Normals are drawn in float32 (``standard_normal(dtype=float32)``), scaled in
float32 and rounded to fp16 (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED = 0
GROUP = 128
PAGE = 16
GLOBAL_LAYER = 1000

# tensor ids
T_QKV_Q, T_QKV_S, T_O_Q, T_O_S = 0, 1, 2, 3
T_GATE_Q, T_GATE_S, T_UP_Q, T_UP_S, T_DOWN_Q, T_DOWN_S = 4, 5, 6, 7, 8, 9
T_LN1, T_LN2, T_BQKV = 10, 11, 12
T_EMBED, T_LMHEAD, T_LNF = 20, 21, 22
T_PROMPT, T_FREELIST = 30, 31
T_X, T_Q, T_K, T_V = 40, 41, 42, 43
T_XM, T_QM = 44, 45


@dataclass(frozen=True)
class ModelDims:
    """Shape constants of a Qwen2.5-7B-style decoder."""
    d_model: int
    d_ff: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    eps: float = 1e-6
    theta: float = 1e6
    page: int = PAGE
    group: int = GROUP

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_dim(self) -> int:
        return self.q_dim + 2 * self.kv_dim


# 28 layers, hidden 3584, MLP 18944, 28 q / 4 kv heads of 128, vocab 152064.
QWEN7B = ModelDims(d_model=3584, d_ff=18944, n_layers=28, n_q_heads=28,
                   n_kv_heads=4, head_dim=128, vocab=152064)
# Small model with the same head_dim / page / group structure, for fast tests.
TINY = ModelDims(d_model=512, d_ff=1024, n_layers=2, n_q_heads=4,
                 n_kv_heads=2, head_dim=128, vocab=1000)


def rng(cfg: int, layer: int, tensor_id: int, seed: int = SEED) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, layer, tensor_id]))


def normal_f16(r: np.random.Generator, shape, scale: float = 1.0, offset: float = 0.0) -> np.ndarray:
    z = r.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        z *= np.float32(scale)
    if offset != 0.0:
        z += np.float32(offset)
    return z.astype(np.float16)


def int4_codes(r: np.random.Generator, n: int, k: int) -> np.ndarray:
    """int8 array [n, k] of signed 4-bit codes, uniform in [-8, 7]."""
    return r.integers(-8, 8, size=(n, k), dtype=np.int8)


def group_scales(r: np.random.Generator, n: int, k: int, group: int = GROUP) -> np.ndarray:
    """fp16 array [n, k // group]: |N(0,1)| * 0.02 + 1e-3."""
    if k % group:
        raise ValueError(f"K={k} is not a multiple of the group size {group}")
    z = np.abs(r.standard_normal((n, k // group), dtype=np.float32))
    z *= np.float32(0.02)
    z += np.float32(1e-3)
    return z.astype(np.float16)


def int4_matrix(cfg: int, layer: int, tid_q: int, tid_s: int, n: int, k: int,
                seed: int = SEED):
    """(codes int8 [n, k], scales fp16 [n, k/128]) from two independent streams."""
    return (int4_codes(rng(cfg, layer, tid_q, seed), n, k),
            group_scales(rng(cfg, layer, tid_s, seed), n, k))


# ----------------------------------------------------------------------------
# kernel-level workloads
# ----------------------------------------------------------------------------

def gemv_case(n: int, k: int, cfg: int = 0, seed: int = SEED, layer: int = GLOBAL_LAYER):
    """One W4A16 GEMV problem: codes [n,k], scales [n,k/128], x fp16 [k]."""
    q, s = int4_matrix(cfg, layer, T_O_Q, T_O_S, n, k, seed)
    x = normal_f16(rng(cfg, layer, T_X, seed), (k,))
    return q, s, x


def gemv_cfg0(seed: int = SEED):
    """Single GEMV, M=1, K=N=3584."""
    return gemv_case(3584, 3584, cfg=0, seed=seed)


def mlp_cfg1(seed: int = SEED, d: int = 3584, f: int = 18944):
    """MLP decode shapes: x [d]; gate, up [f, d]; down [d, f]."""
    cfg = 1
    gq, gs = int4_matrix(cfg, 0, T_GATE_Q, T_GATE_S, f, d, seed)
    uq, us = int4_matrix(cfg, 0, T_UP_Q, T_UP_S, f, d, seed)
    dq, ds = int4_matrix(cfg, 0, T_DOWN_Q, T_DOWN_S, d, f, seed)
    x = normal_f16(rng(cfg, GLOBAL_LAYER, T_X, seed), (d,))
    return dict(x=x, gate=(gq, gs), up=(uq, us), down=(dq, ds))


def attn_case(ctx: int, n_qh: int = 28, n_kvh: int = 4, head_dim: int = 128,
              n_pages: int | None = None, cfg: int = 2, seed: int = SEED,
              shuffle: bool = True):
    """Paged decode attention inputs.

    Returns q fp16 [n_qh, head_dim], K and V pools fp16
    [n_pages, n_kvh, PAGE, head_dim] (physical order), and an int32 page table
    of length ceil(ctx / PAGE) mapping logical page -> physical page.
    """
    need = -(-ctx // PAGE)
    if n_pages is None:
        n_pages = need
    if n_pages < need:
        raise ValueError("pool too small for the context")
    q = normal_f16(rng(cfg, GLOBAL_LAYER, T_Q, seed), (n_qh, head_dim))
    kp = normal_f16(rng(cfg, GLOBAL_LAYER, T_K, seed), (n_pages, n_kvh, PAGE, head_dim))
    vp = normal_f16(rng(cfg, GLOBAL_LAYER, T_V, seed), (n_pages, n_kvh, PAGE, head_dim))
    if shuffle:
        perm = rng(cfg, GLOBAL_LAYER, T_FREELIST, seed).permutation(n_pages)
    else:
        perm = np.arange(n_pages)
    table = perm[:need].astype(np.int32)
    return q, kp, vp, table


def gemm_case(m: int, n: int, k: int, cfg: int = 4, seed: int = SEED, layer: int = GLOBAL_LAYER):
    """One prefill GEMM problem: codes [n,k], scales [n,k/128], X fp16 [m,k]."""
    q, s = int4_matrix(cfg, layer, T_O_Q, T_O_S, n, k, seed)
    x = normal_f16(rng(cfg, layer, T_XM, seed), (m, k))
    return q, s, x


def prefill_attn_case(pos0: int, m: int, n_qh: int = 28, n_kvh: int = 4, head_dim: int = 128,
                      n_pages: int | None = None, cfg: int = 4, seed: int = SEED):
    """Prefill attention inputs: queries fp16 [m, n_qh, head_dim] at positions
    pos0 .. pos0 + m - 1, and paged K/V (shuffled pages) for positions
    0 .. pos0 + m - 1, as in attn_case."""
    _, kp, vp, table = attn_case(pos0 + m, n_qh, n_kvh, head_dim, n_pages, cfg, seed)
    q = normal_f16(rng(cfg, GLOBAL_LAYER, T_QM, seed), (m, n_qh, head_dim))
    return q, kp, vp, table


def attn_cfg2(seed: int = SEED):
    """1 query token, 28 q heads, 4 kv heads, head_dim 128, context 640 in 40 shuffled pages."""
    return attn_case(640, seed=seed)


# ----------------------------------------------------------------------------
# decoder model (random init, Qwen2.5-7B shapes)
# ----------------------------------------------------------------------------

@dataclass
class LayerWeights:
    """One decoder layer.  Projections are (codes int8 [N,K], scales fp16 [N,K/128]).

    QKV rows are ordered [q heads | k heads | v heads], head-major, head_dim
    rows per head.  Norm weights and bias are fp16.
    """
    ln1: np.ndarray
    qkv: tuple
    bqkv: np.ndarray
    o: tuple
    ln2: np.ndarray
    gate: tuple
    up: tuple
    down: tuple


@dataclass
class GlobalWeights:
    embed: np.ndarray    # fp16 [vocab, d]
    lnf: np.ndarray      # fp16 [d]
    lm_head: np.ndarray  # fp16 [vocab, d]


def layer_weights(dims: ModelDims, layer: int, cfg: int = 3, seed: int = SEED) -> LayerWeights:
    d, f = dims.d_model, dims.d_ff
    return LayerWeights(
        ln1=normal_f16(rng(cfg, layer, T_LN1, seed), (d,), 0.1, 1.0),
        qkv=int4_matrix(cfg, layer, T_QKV_Q, T_QKV_S, dims.qkv_dim, d, seed),
        bqkv=normal_f16(rng(cfg, layer, T_BQKV, seed), (dims.qkv_dim,), 0.1),
        o=int4_matrix(cfg, layer, T_O_Q, T_O_S, d, dims.q_dim, seed),
        ln2=normal_f16(rng(cfg, layer, T_LN2, seed), (d,), 0.1, 1.0),
        gate=int4_matrix(cfg, layer, T_GATE_Q, T_GATE_S, f, d, seed),
        up=int4_matrix(cfg, layer, T_UP_Q, T_UP_S, f, d, seed),
        down=int4_matrix(cfg, layer, T_DOWN_Q, T_DOWN_S, d, f, seed),
    )


def global_weights(dims: ModelDims, cfg: int = 3, seed: int = SEED) -> GlobalWeights:
    d, v = dims.d_model, dims.vocab
    return GlobalWeights(
        embed=normal_f16(rng(cfg, GLOBAL_LAYER, T_EMBED, seed), (v, d)),
        lnf=normal_f16(rng(cfg, GLOBAL_LAYER, T_LNF, seed), (d,), 0.1, 1.0),
        lm_head=normal_f16(rng(cfg, GLOBAL_LAYER, T_LMHEAD, seed), (v, d), 0.02),
    )


def prompt_ids(dims: ModelDims, n: int, cfg: int = 3, seed: int = SEED) -> np.ndarray:
    return rng(cfg, GLOBAL_LAYER, T_PROMPT, seed).integers(0, dims.vocab, size=n).astype(np.int32)


def page_free_list(n_pages: int, cfg: int = 3, seed: int = SEED) -> np.ndarray:
    """Physical page handed out for each successive logical page (a permutation)."""
    return rng(cfg, GLOBAL_LAYER, T_FREELIST, seed).permutation(n_pages).astype(np.int32)
