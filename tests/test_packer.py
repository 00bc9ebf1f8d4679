"""Host packer (C++ in libw4a16.so): bit-exact round trip, an independent
decoder written from the layout the header documents, and argument errors.
CPU only."""
import numpy as np
import pytest

import oracle
import synth
import int4_weight_only_dequant_amd as w4
from int4_weight_only_dequant_amd import _lib as L


def decode_layout(pq: np.ndarray, ps: np.ndarray, n: int, k: int):
    """Independent decoder of the packed layout (header of include/w4a16.h).

    16-byte slot of (row block b, chunk c, lane l) at ((b*K/32 + c)*64 + l)*16;
    word d holds elements 32c + 8d + e; element 2j in bits [4j, 4j+4), element
    2j+1 in bits [16+4j, ...); nibble = q + 8.  Scales at (b*K/128 + g)*64 + l.
    """
    nb = -(-n // 64)
    words = pq.view("<u4").reshape(nb, k // 32, 64, 4)             # [b, c, l, d]
    e = np.arange(8)
    shifts = np.where(e % 2 == 0, 4 * (e // 2), 16 + 4 * (e // 2))  # [e]
    nib = (words[..., None] >> shifts.astype(np.uint32)) & 0xF      # [b, c, l, d, e]
    q = nib.astype(np.int16) - 8
    q = q.transpose(0, 2, 1, 3, 4).reshape(nb * 64, k)              # rows, k = 32c + 8d + e
    s = ps.reshape(nb, k // 128, 64).transpose(0, 2, 1).reshape(nb * 64, k // 128)
    return q[:n].astype(np.int8), s[:n].view(np.float16), q[n:], s[n:]


@pytest.mark.parametrize("n,k", [(1, 128), (64, 256), (100, 384), (257, 3584), (70, 18944)])
def test_roundtrip_and_independent_decoder(n, k):
    q, s, _ = synth.gemv_case(n, k, cfg=93)
    pq, ps = w4.pack_int4_weights(q, s)
    assert pq.nbytes == -(-n // 64) * 64 * k // 2
    q2, s2 = w4.unpack_int4_weights(pq, ps, n, k)
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint16), s2.view(np.uint16))
    q3, s3, qpad, spad = decode_layout(pq, ps, n, k)
    assert np.array_equal(q, q3) and np.array_equal(s.view(np.uint16), s3.view(np.uint16))
    assert (qpad == 0).all() and (spad.view(np.uint16) == 0).all()   # pad rows: code 0, scale 0


def test_all_nibbles_and_row_perm():
    n, k = 128, 256
    q = (np.arange(n * k) % 16 - 8).astype(np.int8).reshape(n, k)
    s = np.full((n, k // 128), 0.5, np.float16)
    perm = np.random.default_rng(0).permutation(n).astype(np.int32)
    pq, ps = w4.pack_int4_weights(q, s, row_perm=perm)
    qd, sd, _, _ = decode_layout(pq, ps, n, k)
    assert np.array_equal(qd, q[perm])                    # packed row r holds logical row perm[r]
    q2, _ = w4.unpack_int4_weights(pq, ps, n, k, row_perm=perm)
    assert np.array_equal(q2, q)


def test_model_row_perms():
    cfg = L.ModelConfig(d_model=512, d_ff=1024, n_layers=1, n_q_heads=4, n_kv_heads=2,
                        head_dim=128, vocab=10, max_pages=2, eps=1e-6, theta=1e6)
    p = w4.model_row_perm(L.W4_PERM_QKV, cfg)
    assert p.size == 8 * 128
    assert list(p[:4]) == [0, 64, 1, 65] and list(p[128:130]) == [128, 192]
    assert sorted(p) == list(range(p.size))
    g = w4.model_row_perm(L.W4_PERM_GATE_UP, cfg)
    assert list(g[:4]) == [0, 1024, 1, 1025] and sorted(g) == list(range(2048))


def test_f16_packer_layout():
    w = np.random.default_rng(1).standard_normal((70, 24)).astype(np.float16)
    p = w4.pack_f16_matrix(w).view(np.float16)
    nb = 2
    blk = p.reshape(nb, 24 // 8, 64, 8).transpose(0, 2, 1, 3).reshape(nb * 64, 24)
    assert np.array_equal(blk[:70].view(np.uint16), w.view(np.uint16))
    assert (blk[70:] == 0).all()


def test_pack_errors():
    q, s, _ = synth.gemv_case(8, 256, cfg=93)
    bad = q.copy()
    bad[3, 7] = 8
    with pytest.raises(w4.W4Error) as e:
        w4.pack_int4_weights(bad, s)
    assert e.value.status == L.W4_ERANGE
    s2 = s.copy()
    s2[1, 1] = np.float16(np.nan)
    with pytest.raises(w4.W4Error) as e:
        w4.pack_int4_weights(q, s2)
    assert e.value.status == L.W4_ERANGE
    s3 = s.copy()
    s3[0, 0] = np.float16(np.inf)
    with pytest.raises(w4.W4Error):
        w4.pack_int4_weights(q, s3)
    with pytest.raises(w4.W4Error) as e:
        w4.pack_int4_weights(q, s, row_perm=np.zeros(8, np.int32))
    assert e.value.status == L.W4_EINVAL
    lib = w4.lib()
    assert lib.w4_packed_qbytes(8, 100) == 0 and lib.w4_packed_sbytes(0, 128) == 0
    pq = np.zeros(1 << 12, np.uint8)
    ps = np.zeros(1 << 8, np.uint16)
    assert lib.pack_int4_weights(q.ctypes.data, s.ctypes.data, 8, 256, 64, None, pq.ctypes.data,
                                 ps.ctypes.data) == L.W4_EINVAL          # group != 128
    assert lib.pack_int4_weights(None, s.ctypes.data, 8, 256, 128, None, pq.ctypes.data,
                                 ps.ctypes.data) == L.W4_EALIGN
    assert b"NULL" in lib.w4_last_error()


def test_quantize_int4_weights_matches_oracle_bitexact():
    """The host fp16 -> int4 quantiser equals the oracle's definition bit for
    bit (scales and codes), over several magnitudes, fp16 subnormals, the
    largest fp16, an all-zero group and a group whose scale underflows."""
    r = np.random.default_rng(15)
    w = (r.standard_normal((37, 5 * 128)) * np.repeat([0.02, 1e-5, 500.0, 1.0, 3e-4], 128)).astype(np.float16)
    w[5, 300] = np.float16(-65504.0)
    w[7, 0:128] = 0
    w[9, 128:256] = np.float16(6e-8)
    w[11, 2 * 128 + 5] = np.float16(-1e-7)
    q, s = w4.quantize_int4_weights(w)
    rq, rs = oracle.quantize_int4(w)
    assert np.array_equal(s.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(q, rq)
    # the codes and scales feed the packer unchanged (round trip through the layout)
    pq, ps = w4.pack_int4_weights(q, s)
    q2, s2 = w4.unpack_int4_weights(pq, ps, 37, 5 * 128)
    assert np.array_equal(q2, q) and np.array_equal(s2.view(np.uint16), s.view(np.uint16))


def test_quantize_int4_weights_rejects_bad_input():
    lib = w4.lib()
    w = np.zeros((4, 256), np.float16)
    w[1, 7] = np.float16(np.inf)
    with pytest.raises(L.W4Error) as e:
        w4.quantize_int4_weights(w)
    assert e.value.status == L.W4_ERANGE
    with pytest.raises(L.W4Error):
        w4.quantize_int4_weights(np.zeros((4, 100), np.float16))
    assert lib.quantize_int4_weights(None, 4, 256, 128, None, None) == L.W4_EALIGN
