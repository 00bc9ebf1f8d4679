"""ctypes binding of libw4a16.so (the C ABI declared in include/w4a16.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of the library.  PyTorch provides device memory and streams.  If the
library is missing the calls raise; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import numpy as np
import torch  # imported before the library so both share one HIP runtime

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a16.so")

W4_OK, W4_EINVAL, W4_EALIGN, W4_ERANGE, W4_ESTATE, W4_ENOSPC, W4_EHIP = 0, -1, -2, -3, -4, -5, -6
W4_PERM_QKV, W4_PERM_GATE_UP = 0, 1
W4_GRAPH, W4_EAGER, W4_MULTI, W4_A8 = 0, 1, 2, 4
W4_KERNEL_GATE_UP, W4_KERNEL_DOWN, W4_KERNEL_O, W4_KERNEL_LM_HEAD = 0, 1, 2, 3

_STATUS = {W4_EINVAL: "W4_EINVAL", W4_EALIGN: "W4_EALIGN", W4_ERANGE: "W4_ERANGE",
           W4_ESTATE: "W4_ESTATE", W4_ENOSPC: "W4_ENOSPC", W4_EHIP: "W4_EHIP"}


class W4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class ModelConfig(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("d_ff", C.c_int32), ("n_layers", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("vocab", C.c_int32), ("max_pages", C.c_int32), ("eps", C.c_float),
                ("theta", C.c_double)]


_PP = C.POINTER(C.c_void_p)


class ModelBuffers(C.Structure):
    _fields_ = [(n, _PP) for n in ("qkv_q", "qkv_s", "qkv_bias", "o_q", "o_s", "gu_q", "gu_s",
                                   "down_q", "down_s", "ln1", "ln2")] + \
               [(n, C.c_void_p) for n in ("embed", "lnf", "lm_head", "k_cache", "v_cache",
                                          "page_table", "free_list", "tokens", "logits")]


_lib = None
_lock = threading.Lock()


class W4cTensor(C.Structure):
    _fields_ = [("name", C.c_char_p), ("kind", C.c_int32), ("row_order", C.c_int32), ("rows", C.c_int64),
                ("cols", C.c_int64), ("data", C.c_void_p), ("bytes", C.c_size_t)]


W4_EFORMAT = -7
W4C_INT4_CODES, W4C_INT4_SCALES, W4C_F16, W4C_F16_ROWS = 0, 1, 2, 3


class DebugLayout(C.Structure):
    """w4_debug_layout: where the persistent step keeps its intermediates."""
    _fields_ = [("acc", C.c_void_p * 2), ("acc_layer", C.c_int64), ("acc_q", C.c_int32), ("acc_o", C.c_int32),
                ("acc_gu", C.c_int32), ("acc_d", C.c_int32), ("fix_bits", C.c_int32), ("last_parity", C.c_int32),
                ("resid", C.c_void_p), ("resid_stride", C.c_int64), ("att_part", C.c_void_p),
                ("att_layer_floats", C.c_int64), ("att_smax", C.c_int32), ("att_pages_per_chunk", C.c_int32),
                ("stage_stride", C.c_int32), ("reserved", C.c_int32)]


def _declare(lib):
    vp, i32, i64, sz, u32, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_uint32, C.c_float
    sig = {
        "w4_last_error": (C.c_char_p, []),
        "w4_version": (C.c_char_p, []),
        "w4_packed_qbytes": (sz, [i64, i64]),
        "w4_packed_sbytes": (sz, [i64, i64]),
        "pack_int4_weights": (i32, [vp, vp, i64, i64, i32, vp, vp, vp]),
        "unpack_int4_weights": (i32, [vp, vp, i64, i64, i32, vp, vp, vp]),
        "quantize_int4_weights": (i32, [vp, i64, i64, i32, vp, vp]),
        "w4_packed_f16_bytes": (sz, [i64, i64]),
        "w4_pack_f16_matrix": (i32, [vp, i64, i64, vp]),
        "w4_gemv_ws_bytes": (sz, [i64, i64]),
        "w4a16_gemv": (i32, [vp, vp, vp, vp, i64, i64, vp, sz, vp]),
        "w4_noalloc_scratch_bytes": (sz, []),
        "w4a16_gemv_noalloc": (i32, [vp, vp, vp, vp, i64, i64, vp]),
        "w4c_write": (i32, [C.c_char_p, C.POINTER(ModelConfig), i32, C.POINTER(W4cTensor)]),
        "w4c_open": (i32, [C.c_char_p, C.POINTER(vp)]),
        "w4c_count": (i32, [vp]),
        "w4c_config": (i32, [vp, C.POINTER(ModelConfig)]),
        "w4c_tensor_at": (i32, [vp, i32, C.POINTER(W4cTensor)]),
        "w4c_find": (i32, [vp, C.c_char_p, C.POINTER(W4cTensor)]),
        "w4c_close": (None, [vp]),
        "w4a8_act_bytes": (sz, [i64]),
        "w4a8_quantize_act": (i32, [vp, i64, vp, vp]),
        "w4a8_gemv": (i32, [vp, vp, vp, vp, i64, i64, vp, sz, vp]),
        "w4_mlp_ws_bytes": (sz, [i64, i64]),
        "w4a16_mlp": (i32, [vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, sz, vp]),
        "w4_gemm_ws_bytes": (sz, [i64, i64, i64]),
        "w4a16_gemm": (i32, [vp, vp, vp, vp, i64, i64, i64, vp, sz, vp]),
        "w4_attn_ws_bytes": (sz, [i32, i32, i32]),
        "paged_attn_prefill": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp]),
        "paged_attn_decode": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, sz, vp]),
        "w4_model_row_perm": (i32, [i32, C.POINTER(ModelConfig), vp]),
        "w4_model_create": (i32, [C.POINTER(ModelConfig), C.POINTER(ModelBuffers), C.POINTER(vp)]),
        "w4_model_destroy": (None, [vp]),
        "w4_model_reset": (i32, [vp, i32, vp]),
        "w4_model_pos": (i32, [vp]),
        "decode_step": (i32, [vp, i32, u32, vp]),
        "w4_model_prefill": (i32, [vp, i32, i32, vp]),
        "w4_model_launches_per_step": (i32, [vp, u32]),
        "w4_model_kernel_replay": (i32, [vp, i32, i32, vp]),
        "w4_model_status": (i32, [vp, C.POINTER(i32)]),
        "w4_model_grid": (i32, [vp]),
        "w4_model_debug_layout": (i32, [vp, C.POINTER(DebugLayout)]),
        "w4_model_stage_dump_elems": (sz, [vp]),
        "w4_model_set_stage_dump": (i32, [vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"{LIB_PATH} is not built: run `python -m int4_weight_only_dequant_amd.build`")
                l = C.CDLL(LIB_PATH)
                _declare(l)
                _lib = l
    return _lib


def check(status: int) -> None:
    if status != W4_OK:
        raise W4Error(status, lib().w4_last_error().decode())


def _ptr(a) -> int:
    if isinstance(a, torch.Tensor):
        return a.data_ptr()
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    raise TypeError(type(a))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, dtype_size: int | None = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("expected a CUDA (HIP) torch tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t


# ------------------------------------------------------------------ packing --

def pack_int4_weights(q: np.ndarray, s: np.ndarray, row_perm: np.ndarray | None = None):
    """Host packer: codes int8 [N,K], scales fp16 [N,K/128] -> (packed codes u8, packed scales u16)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float16)
    n, k = q.shape
    L = lib()
    qb, sb = L.w4_packed_qbytes(n, k), L.w4_packed_sbytes(n, k)
    if qb == 0:
        raise W4Error(W4_EINVAL, f"bad shape {q.shape}")
    pq = np.empty(qb, np.uint8)
    ps = np.empty(sb // 2, np.uint16)
    perm = None if row_perm is None else np.ascontiguousarray(row_perm, dtype=np.int32)
    check(L.pack_int4_weights(_ptr(q), _ptr(s), n, k, 128, None if perm is None else _ptr(perm),
                              _ptr(pq), _ptr(ps)))
    return pq, ps


_KIND_DTYPE = {W4C_INT4_CODES: np.uint8, W4C_INT4_SCALES: np.uint16, W4C_F16: np.uint16, W4C_F16_ROWS: np.uint16}


def write_container(path: str, cfg: ModelConfig, tensors) -> None:
    """Writes a weight container; tensors: (name, kind, row_order, rows, cols, numpy array) in file order."""
    keep = []
    arr = (W4cTensor * len(tensors))()
    for i, (name, kind, order, rows, cols, a) in enumerate(tensors):
        a = np.ascontiguousarray(a)
        nm = name.encode()
        keep += [a, nm]
        arr[i] = W4cTensor(nm, kind, order, rows, cols, a.ctypes.data, a.nbytes)
    check(lib().w4c_write(os.fsencode(path), C.byref(cfg), len(tensors), arr))


class Container:
    """A weight container mapped read-only; arrays are views of the mapping,
    valid until close()."""

    def __init__(self, path: str):
        h = C.c_void_p()
        check(lib().w4c_open(os.fsencode(path), C.byref(h)))
        self._h = h

    def config(self) -> ModelConfig:
        cfg = ModelConfig()
        check(lib().w4c_config(self._h, C.byref(cfg)))
        return cfg

    def names(self):
        out = []
        for i in range(lib().w4c_count(self._h)):
            t = W4cTensor()
            check(lib().w4c_tensor_at(self._h, i, C.byref(t)))
            out.append(t.name.decode())
        return out

    def tensor(self, name: str):
        """(kind, row_order, rows, cols, numpy view of the bytes)."""
        t = W4cTensor()
        check(lib().w4c_find(self._h, name.encode(), C.byref(t)))
        dt = np.dtype(_KIND_DTYPE[t.kind])
        buf = (C.c_char * t.bytes).from_address(t.data)
        return t.kind, t.row_order, t.rows, t.cols, np.frombuffer(buf, dtype=dt)

    def close(self) -> None:
        if self._h:
            lib().w4c_close(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def quantize_int4_weights(w: np.ndarray):
    """Host quantiser: fp16 weights [N, K] -> (codes int8 [N, K], scales fp16 [N, K/128])."""
    w = np.ascontiguousarray(w, dtype=np.float16)
    n, k = w.shape
    q = np.empty((n, k), np.int8)
    s = np.empty((n, max(k // 128, 1)), np.float16)
    check(lib().quantize_int4_weights(_ptr(w), n, k, 128, _ptr(q), _ptr(s)))
    return q, s


def unpack_int4_weights(pq: np.ndarray, ps: np.ndarray, n: int, k: int,
                        row_perm: np.ndarray | None = None):
    q = np.empty((n, k), np.int8)
    s = np.empty((n, k // 128), np.float16)
    perm = None if row_perm is None else np.ascontiguousarray(row_perm, dtype=np.int32)
    check(lib().unpack_int4_weights(_ptr(np.ascontiguousarray(pq)), _ptr(np.ascontiguousarray(ps)), n, k, 128,
                                    None if perm is None else _ptr(perm), _ptr(q), _ptr(s)))
    return q, s


def pack_f16_matrix(w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float16)
    n, k = w.shape
    nb = lib().w4_packed_f16_bytes(n, k)
    if nb == 0:
        raise W4Error(W4_EINVAL, f"bad shape {w.shape}")
    out = np.empty(nb // 2, np.uint16)
    check(lib().w4_pack_f16_matrix(_ptr(w), n, k, _ptr(out)))
    return out


def model_row_perm(kind: int, cfg: ModelConfig) -> np.ndarray:
    if kind == W4_PERM_QKV:
        n = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    else:
        n = 2 * cfg.d_ff
    perm = np.empty(n, np.int32)
    check(lib().w4_model_row_perm(kind, C.byref(cfg), _ptr(perm)))
    return perm


# ------------------------------------------------------------- GPU kernels --

_ws_cache: dict = {}


def _workspace(kind: str, nbytes: int, device: torch.device, stream: int) -> torch.Tensor:
    """Scratch buffer per (entry point, device, stream), grown on demand.  It
    starts zeroed: the calls need a zero workspace and leave it zero."""
    key = (kind, device.index, stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def w4a16_gemv(packed_q: torch.Tensor, packed_s: torch.Tensor, x: torch.Tensor, n: int, k: int,
               y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = fp16(W x) for a packed int4 matrix (rows in packed order)."""
    _dev(packed_q), _dev(packed_s), _dev(x)
    if x.dtype != torch.float16 or x.numel() != k:
        raise ValueError("x must be fp16 of length K")
    L = lib()
    if packed_q.numel() * packed_q.element_size() < L.w4_packed_qbytes(n, k):
        raise ValueError("packed codes too small for N x K")
    if packed_s.numel() * packed_s.element_size() < L.w4_packed_sbytes(n, k):
        raise ValueError("packed scales too small for N x K")
    if y is None:
        y = torch.empty(n, dtype=torch.float16, device=x.device)
    _dev(y)
    st = _stream(stream)
    need = L.w4_gemv_ws_bytes(n, k)
    ws = _workspace("gemv", need, x.device, st)
    check(L.w4a16_gemv(_ptr(packed_q), _ptr(packed_s), _ptr(x), _ptr(y), n, k, _ptr(ws),
                       ws.numel(), st))
    return y


def w4a16_gemv_noalloc(packed_q: torch.Tensor, packed_s: torch.Tensor, x: torch.Tensor, y: torch.Tensor,
                       n: int, k: int, stream=None) -> None:
    """w4a16_gemv into a caller-given y, with the library's fixed workspace
    (the call allocates nothing)."""
    _dev(packed_q), _dev(packed_s), _dev(x), _dev(y)
    if x.dtype != torch.float16 or x.numel() != k or y.dtype != torch.float16 or y.numel() < n:
        raise ValueError("x must be fp16 of length K, y fp16 of length >= N")
    L = lib()
    if packed_q.numel() * packed_q.element_size() < L.w4_packed_qbytes(n, k):
        raise ValueError("packed codes too small for N x K")
    if packed_s.numel() * packed_s.element_size() < L.w4_packed_sbytes(n, k):
        raise ValueError("packed scales too small for N x K")
    check(L.w4a16_gemv_noalloc(_ptr(packed_q), _ptr(packed_s), _ptr(x), _ptr(y), n, k, _stream(stream)))


def w4a8_quantize_act(x: torch.Tensor, act: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Int8 activation buffer (codes, group scales and code sums; layout in
    include/w4a16.h) of an fp16 vector x [K]."""
    _dev(x)
    if x.dtype != torch.float16 or x.dim() != 1:
        raise ValueError("x must be a 1-D fp16 tensor")
    L = lib()
    need = L.w4a8_act_bytes(x.numel())
    if need == 0:
        raise ValueError("K must be a positive multiple of 128")
    if act is None:
        act = torch.empty(need, dtype=torch.uint8, device=x.device)
    _dev(act)
    if act.numel() * act.element_size() < need:
        raise ValueError("activation buffer too small")
    check(L.w4a8_quantize_act(_ptr(x), x.numel(), _ptr(act), _stream(stream)))
    return act


def w4a8_gemv(packed_q: torch.Tensor, packed_s: torch.Tensor, act: torch.Tensor, n: int, k: int,
              y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = fp16(W x) with int8 activations from w4a8_quantize_act (rows in packed order)."""
    _dev(packed_q), _dev(packed_s), _dev(act)
    L = lib()
    if act.numel() * act.element_size() < L.w4a8_act_bytes(k):
        raise ValueError("activation buffer too small for K")
    if packed_q.numel() * packed_q.element_size() < L.w4_packed_qbytes(n, k):
        raise ValueError("packed codes too small for N x K")
    if packed_s.numel() * packed_s.element_size() < L.w4_packed_sbytes(n, k):
        raise ValueError("packed scales too small for N x K")
    if y is None:
        y = torch.empty(n, dtype=torch.float16, device=act.device)
    _dev(y)
    st = _stream(stream)
    need = L.w4_gemv_ws_bytes(n, k)
    ws = _workspace("gemv", need, act.device, st)
    check(L.w4a8_gemv(_ptr(packed_q), _ptr(packed_s), _ptr(act), _ptr(y), n, k, _ptr(ws), ws.numel(), st))
    return y


def w4a16_mlp(gu_q: torch.Tensor, gu_s: torch.Tensor, down_q: torch.Tensor, down_s: torch.Tensor,
              x: torch.Tensor, d: int, f: int, stream=None):
    """MLP block of one token: (h, y) with h = fp16(silu(Wg x) * Wu x), y = fp16(Wd h).

    gu_q/gu_s: [gate; up] packed with the W4_PERM_GATE_UP row order."""
    for t in (gu_q, gu_s, down_q, down_s, x):
        _dev(t)
    if x.dtype != torch.float16 or x.numel() != d:
        raise ValueError("x must be fp16 of length D")
    L = lib()
    if gu_q.numel() * gu_q.element_size() < L.w4_packed_qbytes(2 * f, d) or \
            down_q.numel() * down_q.element_size() < L.w4_packed_qbytes(d, f):
        raise ValueError("packed weights too small")
    h = torch.empty(f, dtype=torch.float16, device=x.device)
    y = torch.empty(d, dtype=torch.float16, device=x.device)
    st = _stream(stream)
    need = L.w4_mlp_ws_bytes(d, f)
    ws = _workspace("mlp", need, x.device, st)
    check(L.w4a16_mlp(_ptr(gu_q), _ptr(gu_s), _ptr(down_q), _ptr(down_s), _ptr(x), _ptr(h), _ptr(y),
                      d, f, _ptr(ws), ws.numel(), st))
    return h, y


def w4a16_gemm(packed_q: torch.Tensor, packed_s: torch.Tensor, x: torch.Tensor, n: int, k: int,
               y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X W^T (fp32 [M, N]) for fp16 rows X [M, K] and a packed int4 matrix (rows in packed order)."""
    _dev(packed_q), _dev(packed_s), _dev(x)
    if x.dtype != torch.float16 or x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be fp16 [M, K]")
    m = x.shape[0]
    L = lib()
    if packed_q.numel() * packed_q.element_size() < L.w4_packed_qbytes(n, k):
        raise ValueError("packed codes too small for N x K")
    if packed_s.numel() * packed_s.element_size() < L.w4_packed_sbytes(n, k):
        raise ValueError("packed scales too small for N x K")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(y)
    st = _stream(stream)
    need = L.w4_gemm_ws_bytes(m, n, k)
    ws = _workspace("gemm", need, x.device, st)
    check(L.w4a16_gemm(_ptr(packed_q), _ptr(packed_s), _ptr(x), _ptr(y), m, n, k, _ptr(ws),
                       ws.numel(), st))
    return y


def paged_attn_prefill(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                       page_table: torch.Tensor, pos0: int, scale: float,
                       out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Causal attention of M prompt tokens at positions pos0.. over the paged cache (fp16 in/out)."""
    for t in (q, k_pool, v_pool, page_table):
        _dev(t)
    m, n_qh, hd = q.shape
    n_phys, n_kvh, page, hd2 = k_pool.shape
    if page != 16 or hd2 != hd or v_pool.shape != k_pool.shape:
        raise ValueError("pools must be [n_phys, n_kvh, 16, head_dim]")
    if page_table.dtype != torch.int32 or page_table.numel() * 16 < pos0 + m:
        raise ValueError("page_table must be int32 and cover every position < pos0 + M")
    if out is None:
        out = torch.empty_like(q)
    _dev(out)
    check(lib().paged_attn_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table), int(pos0),
                                   m, n_qh, n_kvh, hd, float(scale), _ptr(out), _stream(stream)))
    return out


def paged_attn_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                      page_table: torch.Tensor, ctx_len: int, scale: float,
                      out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode attention of one token over ctx_len paged tokens (fp16 in, fp16 out)."""
    for t in (q, k_pool, v_pool, page_table):
        _dev(t)
    n_qh, hd = q.shape
    n_phys, n_kvh, page, hd2 = k_pool.shape
    if page != 16 or hd2 != hd or v_pool.shape != k_pool.shape:
        raise ValueError("pools must be [n_phys, n_kvh, 16, head_dim]")
    if page_table.dtype != torch.int32:
        raise ValueError("page_table must be int32")
    if out is None:
        out = torch.empty_like(q)
    _dev(out)
    n_pages_max = page_table.numel()
    L = lib()
    st = _stream(stream)
    need = L.w4_attn_ws_bytes(n_qh, n_kvh, n_pages_max)
    ws = _workspace("attn", need, q.device, st)
    check(L.paged_attn_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table), int(ctx_len),
                              n_qh, n_kvh, hd, n_pages_max, float(scale), _ptr(out), _ptr(ws),
                              ws.numel(), st))
    return out


__all__ = [n for n in dir() if not n.startswith("_")]
