"""Decoder model on the GPU: packs synthetic weights, uploads them, and drives
the library's graph-captured decode step.  Marshalling only; every step of the
decode runs in libw4a16's kernels."""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib as L


def _to_dev(a: np.ndarray, device) -> torch.Tensor:
    """Upload raw bytes of a numpy array (fp16 travels as int16 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16 or a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


LAYER_NAMES = ("qkv_q", "qkv_s", "qkv_bias", "o_q", "o_s", "gu_q", "gu_s", "down_q", "down_s", "ln1", "ln2")


def _config(dims, max_pages: int) -> L.ModelConfig:
    return L.ModelConfig(d_model=dims.d_model, d_ff=dims.d_ff, n_layers=dims.n_layers,
                         n_q_heads=dims.n_q_heads, n_kv_heads=dims.n_kv_heads,
                         head_dim=dims.head_dim, vocab=dims.vocab, max_pages=max_pages,
                         eps=dims.eps, theta=dims.theta)


def _pack_layer(lw, perm_qkv, perm_gu) -> dict:
    """One layer's tensors in the layout the library reads (packed projections in
    the model's row orders, fp16 bias and norm weights)."""
    pq, ps = L.pack_int4_weights(*lw.qkv, row_perm=perm_qkv)
    parts = {"qkv_q": pq, "qkv_s": ps, "qkv_bias": lw.bqkv, "ln1": lw.ln1, "ln2": lw.ln2}
    parts["o_q"], parts["o_s"] = L.pack_int4_weights(*lw.o)
    gq = np.concatenate([lw.gate[0], lw.up[0]])
    gs = np.concatenate([lw.gate[1], lw.up[1]])
    parts["gu_q"], parts["gu_s"] = L.pack_int4_weights(gq, gs, row_perm=perm_gu)
    parts["down_q"], parts["down_s"] = L.pack_int4_weights(*lw.down)
    return parts


def _layer_shapes(dims) -> dict:
    """(kind, row order, rows, cols) of each layer tensor (logical shapes)."""
    qkv = (dims.n_q_heads + 2 * dims.n_kv_heads) * dims.head_dim
    qd = dims.n_q_heads * dims.head_dim
    return {"qkv_q": (L.W4C_INT4_CODES, 1 + L.W4_PERM_QKV, qkv, dims.d_model),
            "qkv_s": (L.W4C_INT4_SCALES, 1 + L.W4_PERM_QKV, qkv, dims.d_model),
            "qkv_bias": (L.W4C_F16, 0, 1, qkv),
            "o_q": (L.W4C_INT4_CODES, 0, dims.d_model, qd), "o_s": (L.W4C_INT4_SCALES, 0, dims.d_model, qd),
            "gu_q": (L.W4C_INT4_CODES, 1 + L.W4_PERM_GATE_UP, 2 * dims.d_ff, dims.d_model),
            "gu_s": (L.W4C_INT4_SCALES, 1 + L.W4_PERM_GATE_UP, 2 * dims.d_ff, dims.d_model),
            "down_q": (L.W4C_INT4_CODES, 0, dims.d_model, dims.d_ff),
            "down_s": (L.W4C_INT4_SCALES, 0, dims.d_model, dims.d_ff),
            "ln1": (L.W4C_F16, 0, 1, dims.d_model), "ln2": (L.W4C_F16, 0, 1, dims.d_model)}


def write_model_container(path: str, dims, layer_fn, glob) -> None:
    """Packs a model (layer_fn(l) -> LayerWeights, glob -> GlobalWeights) into a
    weight container at path."""
    cfg = _config(dims, 0)
    perm_qkv = L.model_row_perm(L.W4_PERM_QKV, cfg)
    perm_gu = L.model_row_perm(L.W4_PERM_GATE_UP, cfg)
    shapes = _layer_shapes(dims)
    tensors = []
    for l in range(dims.n_layers):
        parts = _pack_layer(layer_fn(l), perm_qkv, perm_gu)
        for n in LAYER_NAMES:
            kind, order, rows, cols = shapes[n]
            tensors.append((f"layer{l}.{n}", kind, order, rows, cols, parts[n]))
    tensors.append(("embed", L.W4C_F16, 0, dims.vocab, dims.d_model, glob.embed))
    tensors.append(("lnf", L.W4C_F16, 0, 1, dims.d_model, glob.lnf))
    tensors.append(("lm_head", L.W4C_F16_ROWS, 0, dims.vocab, dims.d_model, L.pack_f16_matrix(glob.lm_head)))
    L.write_container(path, cfg, tensors)


class _Dims:
    """Model shape read back from a container's config."""

    def __init__(self, cfg: L.ModelConfig):
        for f, _ in L.ModelConfig._fields_:
            setattr(self, f, getattr(cfg, f))
        self.eps = float(np.float32(cfg.eps))


class DecodeModel:
    """A Qwen2.5-7B-shaped decoder held in device memory.

    dims: a ``synth.ModelDims``; layer_fn(l) returns the layer's LayerWeights
    (codes, scales and fp16 tensors as numpy arrays); glob the GlobalWeights;
    free_list the physical page for each successive logical page.
    ``DecodeModel.from_container`` builds the same model from a weight
    container's mapped, already packed tensors.
    """

    def __init__(self, dims, layer_fn, glob, free_list: np.ndarray, max_pages: int,
                 device="cuda", progress=None):
        cfg = _config(dims, max_pages)
        perm_qkv = L.model_row_perm(L.W4_PERM_QKV, cfg)
        perm_gu = L.model_row_perm(L.W4_PERM_GATE_UP, cfg)
        layers = (_pack_layer(layer_fn(l), perm_qkv, perm_gu) for l in range(dims.n_layers))
        self._build(dims, cfg, layers, glob.embed, glob.lnf, L.pack_f16_matrix(glob.lm_head), free_list,
                    max_pages, device, progress)

    @classmethod
    def from_container(cls, path: str, free_list: np.ndarray, max_pages: int, device="cuda", progress=None):
        c = L.Container(path)
        try:
            dims = _Dims(c.config())
            cfg = _config(dims, max_pages)
            layers = ({n: c.tensor(f"layer{l}.{n}")[4] for n in LAYER_NAMES} for l in range(dims.n_layers))
            self = cls.__new__(cls)
            self._build(dims, cfg, layers, c.tensor("embed")[4], c.tensor("lnf")[4], c.tensor("lm_head")[4],
                        free_list, max_pages, device, progress)
        finally:
            c.close()                    # every tensor has been copied to the device
        return self

    def _build(self, dims, cfg, layers, embed, lnf, lm_head_packed, free_list, max_pages, device, progress):
        self.dims = dims
        self.device = torch.device(device)
        self.cfg = cfg
        self.max_pages = max_pages
        keep = []                        # device tensors must outlive the model
        ptrs = {n: [] for n in LAYER_NAMES}
        dev = self.device
        for l, parts in enumerate(layers):
            for n in LAYER_NAMES:
                t = _to_dev(parts[n], dev)
                keep.append(t)
                ptrs[n].append(t.data_ptr())
            del parts
            if progress:
                progress(l)
        self.embed = _to_dev(embed, dev)
        self.lnf = _to_dev(lnf, dev)
        self.lm_head = _to_dev(lm_head_packed, dev)
        kv_elems = dims.n_layers * max_pages * dims.n_kv_heads * 16 * dims.head_dim
        self.k_cache = torch.zeros(kv_elems, dtype=torch.float16, device=dev)
        self.v_cache = torch.zeros(kv_elems, dtype=torch.float16, device=dev)
        fl = np.ascontiguousarray(free_list, dtype=np.int32)
        # the step writes K/V rows to the pages the free list hands out: an
        # entry outside the pool would be a write out of bounds
        if fl.shape != (max_pages,) or not np.array_equal(np.sort(fl), np.arange(max_pages, dtype=np.int32)):
            raise L.W4Error(L.W4_EINVAL, f"free_list must be a permutation of [0, {max_pages})")
        self.page_table = torch.full((max_pages,), -1, dtype=torch.int32, device=dev)
        self.free_list = torch.from_numpy(fl).to(dev)
        self.tokens = torch.zeros(16 * max_pages + 1, dtype=torch.int32, device=dev)
        self.logits = torch.zeros(dims.vocab, dtype=torch.float32, device=dev)
        self._keep = keep
        self._arrays = {n: (C.c_void_p * dims.n_layers)(*ptrs[n]) for n in LAYER_NAMES}
        buf = L.ModelBuffers()
        for n in LAYER_NAMES:
            setattr(buf, n, C.cast(self._arrays[n], C.POINTER(C.c_void_p)))
        buf.embed, buf.lnf, buf.lm_head = self.embed.data_ptr(), self.lnf.data_ptr(), self.lm_head.data_ptr()
        buf.k_cache, buf.v_cache = self.k_cache.data_ptr(), self.v_cache.data_ptr()
        buf.page_table, buf.free_list = self.page_table.data_ptr(), self.free_list.data_ptr()
        buf.tokens, buf.logits = self.tokens.data_ptr(), self.logits.data_ptr()
        self._buf = buf
        torch.cuda.synchronize(dev)
        handle = C.c_void_p()
        L.check(L.lib().w4_model_create(C.byref(cfg), C.byref(buf), C.byref(handle)))
        self._m = handle

    # ------------------------------------------------------------------
    def reset(self, prompt: np.ndarray, stream=None) -> None:
        prompt = np.ascontiguousarray(prompt, dtype=np.int32)
        # token ids index the embedding rows; the pool bounds the positions
        if prompt.ndim != 1 or len(prompt) < 1 or len(prompt) > 16 * self.max_pages:
            raise L.W4Error(L.W4_EINVAL, f"prompt must hold 1..{16 * self.max_pages} token ids")
        if prompt.min() < 0 or prompt.max() >= self.dims.vocab:
            raise L.W4Error(L.W4_EINVAL, f"prompt token ids must lie in [0, {self.dims.vocab})")
        self.tokens.zero_()
        self.tokens[: len(prompt)] = torch.from_numpy(prompt).to(self.device)
        self.page_table.fill_(-1)
        L.check(L.lib().w4_model_reset(self._m, len(prompt), L._stream(stream)))

    @property
    def pos(self) -> int:
        return L.lib().w4_model_pos(self._m)

    def step(self, flags: int = L.W4_GRAPH, stream=None) -> None:
        decode_step(self, self.pos, flags, stream)

    def prefill(self, n_tokens: int, stream=None) -> None:
        """Prefill n_tokens positions from the current one (one call, up to 512 tokens)."""
        prefill(self, self.pos, n_tokens, stream)

    def device_error(self) -> int:
        """Synchronise and return the persistent step's error word (0 = ok)."""
        v = C.c_int32()
        L.check(L.lib().w4_model_status(self._m, C.byref(v)))
        return v.value

    def debug_layout(self) -> "L.DebugLayout":
        """Where the persistent step keeps its per-layer intermediates (synchronises)."""
        out = L.DebugLayout()
        L.check(L.lib().w4_model_debug_layout(self._m, C.byref(out)))
        return out

    def set_stage_dump(self, on: bool) -> None:
        """Turn the staged-input dump of later persistent steps on or off; the
        buffer (fp16, [4 n_layers + 1][stage_stride]) is self.stage_dump."""
        if on:
            n = L.lib().w4_model_stage_dump_elems(self._m)
            self.stage_dump = torch.zeros(n, dtype=torch.float16, device=self.device)
            L.check(L.lib().w4_model_set_stage_dump(self._m, self.stage_dump.data_ptr()))
        else:
            L.check(L.lib().w4_model_set_stage_dump(self._m, None))
            self.stage_dump = None

    def grid(self) -> int:
        return L.lib().w4_model_grid(self._m)

    def launches_per_step(self, flags: int = 0) -> int:
        """Kernel launches of one step of the given variant (page append not counted)."""
        return L.lib().w4_model_launches_per_step(self._m, flags)

    def kernel_replay(self, kind: int, reps: int, stream=None) -> None:
        """Enqueue reps launches of one step kernel (timing hook; scratch is clobbered)."""
        L.check(L.lib().w4_model_kernel_replay(self._m, kind, reps, L._stream(stream)))

    def close(self) -> None:
        if getattr(self, "_m", None):
            L.lib().w4_model_destroy(self._m)
            self._m = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def decode_step(model: DecodeModel, pos: int, flags: int = L.W4_GRAPH, stream=None) -> None:
    """One decode step at position pos (graph replay by default)."""
    L.check(L.lib().decode_step(model._m, int(pos), int(flags), L._stream(stream)))


def prefill(model: DecodeModel, pos: int, n_tokens: int, stream=None) -> None:
    """Prefill tokens[pos : pos + n_tokens] (logits of the last one, greedy token after it)."""
    L.check(L.lib().w4_model_prefill(model._m, int(pos), int(n_tokens), L._stream(stream)))
