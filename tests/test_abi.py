"""The C-ABI library loads and exports every function include/w4a16.h
declares; argument errors are rejected on the host (no GPU work)."""
import os
import re

import numpy as np

import int4_weight_only_dequant_amd as w4
from int4_weight_only_dequant_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "w4a16.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"pack_int4_weights", "w4a16_gemv", "paged_attn_decode", "decode_step",
            "w4a16_mlp", "w4_model_create"} <= set(names)
    lib = w4.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_no_undefined_library_symbols():
    """Every symbol of the library's own namespace is defined in it (a kernel
    launched from host code whose launch stub was not emitted would otherwise
    surface only when the library is loaded)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        import pytest
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", L.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    ours = [l.split()[-1] for l in out.splitlines() if "2w4" in l or "w4a16" in l or "w4_" in l]
    assert not ours, ours


def test_host_side_argument_errors():
    lib = w4.lib()
    buf = np.zeros(1 << 16, np.uint8)
    p = buf.ctypes.data + (-buf.ctypes.data % 16)
    # K not a multiple of 128
    assert lib.w4a16_gemv(p, p, p, p, 64, 100, p, 4096, None) == L.W4_EINVAL
    # misaligned x
    assert lib.w4a16_gemv(p, p, p + 2, p, 64, 128, p, 4096, None) == L.W4_EALIGN
    # workspace too small
    assert lib.w4a16_gemv(p, p, p, p, 4096, 3584, p, 16, None) == L.W4_EINVAL
    assert lib.w4_gemv_ws_bytes(3584, 3584) > 0 and lib.w4_gemv_ws_bytes(3584, 100) == 0
    # int8 activations: K, alignment, workspace
    assert lib.w4a8_act_bytes(100) == 0 and lib.w4a8_act_bytes(3584) >= 3584 + 2 * 4 * 28
    assert lib.w4a8_quantize_act(p, 100, p, None) == L.W4_EINVAL
    assert lib.w4a8_quantize_act(p + 2, 128, p, None) == L.W4_EALIGN
    assert lib.w4a8_gemv(p, p, p, p, 64, 100, p, 4096, None) == L.W4_EINVAL
    assert lib.w4a8_gemv(p, p, p + 4, p, 64, 128, p, 4096, None) == L.W4_EALIGN
    assert lib.w4a8_gemv(p, p, p, p, 4096, 3584, p, 16, None) == L.W4_EINVAL
    # attention: head_dim, GQA ratio, context range
    assert lib.paged_attn_decode(p, p, p, p, 10, 28, 4, 64, 40, 0.1, p, p, 1 << 15, None) == L.W4_EINVAL
    assert lib.paged_attn_decode(p, p, p, p, 10, 12, 4, 128, 40, 0.1, p, p, 1 << 15, None) == L.W4_EINVAL
    assert lib.paged_attn_decode(p, p, p, p, 641, 28, 4, 128, 40, 0.1, p, p, 1 << 16, None) == L.W4_EINVAL
    assert lib.paged_attn_decode(p, p, p, p, 0, 28, 4, 128, 40, 0.1, p, p, 1 << 16, None) == L.W4_EINVAL
    assert lib.w4a16_mlp(p, p, p, p, p, p, p, 100, 256, p, 1 << 16, None) == L.W4_EINVAL
    # prefill GEMM: K, M range, alignment, workspace
    assert lib.w4a16_gemm(p, p, p, p, 64, 256, 100, p, 1 << 16, None) == L.W4_EINVAL
    assert lib.w4a16_gemm(p, p, p, p, 0, 256, 128, p, 1 << 16, None) == L.W4_EINVAL
    assert lib.w4a16_gemm(p, p, p + 2, p, 64, 256, 128, p, 1 << 16, None) == L.W4_EALIGN
    assert lib.w4a16_gemm(p, p, p, p, 512, 3584, 3584, p, 16, None) == L.W4_EINVAL
    assert lib.w4_gemm_ws_bytes(512, 3584, 3584) >= 4 * 512 * 3584 and lib.w4_gemm_ws_bytes(1, 64, 100) == 0
    # prefill attention: head_dim, head ratio, token count, scale
    assert lib.paged_attn_prefill(p, p, p, p, 0, 16, 28, 4, 64, 0.1, p, None) == L.W4_EINVAL
    assert lib.paged_attn_prefill(p, p, p, p, 0, 16, 12, 8, 128, 0.1, p, None) == L.W4_EINVAL
    assert lib.paged_attn_prefill(p, p, p, p, 0, 0, 28, 4, 128, 0.1, p, None) == L.W4_EINVAL
    assert lib.paged_attn_prefill(p, p, p, p, 0, 16, 28, 4, 128, 0.0, p, None) == L.W4_EINVAL
    assert lib.paged_attn_prefill(p, p + 2, p, p, 0, 16, 28, 4, 128, 0.1, p, None) == L.W4_EALIGN
    # model calls without a model
    assert lib.w4_model_prefill(None, 0, 16, None) == L.W4_ESTATE
    assert lib.decode_step(None, 0, 0, None) == L.W4_ESTATE
    assert lib.w4_model_reset(None, 1, None) == L.W4_ESTATE
    assert lib.w4_model_pos(None) == -1
