"""Weight container: round trip of a packed tiny model and fail-fast refusal of
damaged files (host-side; no GPU work)."""
import os
import struct

import numpy as np
import pytest

import synth
import int4_weight_only_dequant_amd as w4
from int4_weight_only_dequant_amd import _lib as L
from int4_weight_only_dequant_amd import model as M

DIMS = synth.TINY


@pytest.fixture(scope="module")
def container(tmp_path_factory):
    path = str(tmp_path_factory.mktemp("w4c") / "tiny.w4c")
    layers = [synth.layer_weights(DIMS, l, cfg=120) for l in range(DIMS.n_layers)]
    glob = synth.global_weights(DIMS, cfg=120)
    M.write_model_container(path, DIMS, lambda l: layers[l], glob)
    return path, layers, glob


def test_round_trip(container):
    path, layers, glob = container
    c = L.Container(path)
    try:
        cfg = c.config()
        assert (cfg.d_model, cfg.d_ff, cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.vocab) == \
            (DIMS.d_model, DIMS.d_ff, DIMS.n_layers, DIMS.n_q_heads, DIMS.n_kv_heads, DIMS.head_dim, DIMS.vocab)
        names = c.names()
        assert names == [f"layer{l}.{n}" for l in range(DIMS.n_layers) for n in M.LAYER_NAMES] + \
            ["embed", "lnf", "lm_head"]
        cf = M._config(DIMS, 0)
        perm_qkv = L.model_row_perm(L.W4_PERM_QKV, cf)
        perm_gu = L.model_row_perm(L.W4_PERM_GATE_UP, cf)
        for l in range(DIMS.n_layers):
            parts = M._pack_layer(layers[l], perm_qkv, perm_gu)
            for n in M.LAYER_NAMES:
                kind, order, rows, cols, arr = c.tensor(f"layer{l}.{n}")
                want = np.ascontiguousarray(parts[n])
                assert arr.tobytes() == want.tobytes(), (l, n)
                assert (kind, order, rows, cols) == M._layer_shapes(DIMS)[n]
        assert c.tensor("embed")[4].tobytes() == glob.embed.tobytes()
        assert c.tensor("lm_head")[4].tobytes() == L.pack_f16_matrix(glob.lm_head).tobytes()
        # every tensor starts on a 4096-byte boundary of the file
        raw = open(path, "rb").read()
        n_t = struct.unpack_from("<I", raw, 16)[0]
        for i in range(n_t):
            off = struct.unpack_from("<Q", raw, 256 + 96 * i + 72)[0]
            assert off % 4096 == 0
    finally:
        c.close()


def _damaged(path, tmp_path, edit):
    raw = bytearray(open(path, "rb").read())
    raw = edit(raw)
    out = str(tmp_path / "bad.w4c")
    with open(out, "wb") as fh:
        fh.write(raw)
    return out


@pytest.mark.parametrize("what,edit", [
    ("bad magic", lambda r: r.__setitem__(0, ord("X")) or r),
    ("the pages' magic", lambda r: r.__setitem__(slice(0, 8), b"NANOQWEN") or r),
    ("version", lambda r: r.__setitem__(slice(8, 12), struct.pack("<I", 2)) or r),
    ("truncated", lambda r: r[:-4096]),
    ("padded", lambda r: r + bytes(4096)),
    ("table byte", lambda r: r.__setitem__(256 + 50, r[256 + 50] ^ 1) or r),
    ("shorter than a header", lambda r: r[:100]),
])
def test_damaged_files_are_refused(container, tmp_path, what, edit):
    path = _damaged(container[0], tmp_path, edit)
    with pytest.raises(L.W4Error) as e:
        L.Container(path)
    assert e.value.status == L.W4_EFORMAT, what


def _fnv1a64(b: bytes) -> int:
    h = 1469598103934665603
    for c in b:
        h = ((h ^ c) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h


def test_wrapped_tensor_offset_is_refused(container, tmp_path):
    """An entry whose offset + size wraps past 2^64 (table checksum recomputed,
    so only the bounds check stands in the way) is refused."""
    def edit(r):
        n_t = struct.unpack_from("<I", r, 16)[0]
        last = 256 + 96 * (n_t - 1)
        nbytes = struct.unpack_from("<Q", r, last + 80)[0]
        assert nbytes > 4096                               # so the sum really wraps
        struct.pack_into("<Q", r, last + 72, (1 << 64) - 4096)
        struct.pack_into("<Q", r, 40, _fnv1a64(bytes(r[256:256 + 96 * n_t])))
        return r
    path = _damaged(container[0], tmp_path, edit)
    with pytest.raises(L.W4Error) as e:
        L.Container(path)
    assert e.value.status == L.W4_EFORMAT
    assert "bounds" in str(e.value)


def test_open_and_write_errors(tmp_path):
    with pytest.raises(L.W4Error) as e:
        L.Container(str(tmp_path / "missing.w4c"))
    assert e.value.status == L.W4_EINVAL
    cfg = M._config(DIMS, 0)
    with pytest.raises(L.W4Error):       # byte count does not match the kind and shape
        L.write_container(str(tmp_path / "x.w4c"), cfg,
                          [("t", L.W4C_INT4_CODES, 0, 64, 128, np.zeros(100, np.uint8))])
