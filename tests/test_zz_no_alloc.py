"""The allocation-free GEMV entry point (w4a16_gemv_noalloc) against the
workspace entry point (w4a16_gemv): bit-identical outputs, on two calls in a
row, the second smaller, and within the GEMV tolerance of the oracle; shapes
beyond its fixed workspace are refused."""
import numpy as np
import pytest
import torch

import oracle
import synth
import int4_weight_only_dequant_amd as w4
from int4_weight_only_dequant_amd import _lib as L
from tests._tol import assert_gemv

pytestmark = pytest.mark.gpu


def _case(n, k, cfg):
    q, s, x = synth.gemv_case(n, k, cfg=cfg)
    pq, ps = w4.pack_int4_weights(q, s)
    dev = torch.device("cuda")
    return (q, s, x, torch.from_numpy(pq).to(dev), torch.from_numpy(ps.view(np.int16)).to(dev),
            torch.from_numpy(x).to(dev))


def test_noalloc_gemv_equals_workspace_gemv_twice():
    print("case: w4a16_gemv_noalloc 37888x3584 then 3584x18944 then 3584x3584", flush=True)
    for n, k, cfg in ((37888, 3584, 140), (3584, 18944, 141), (3584, 3584, 142), (200, 256, 143)):
        q, s, x, pq, ps, xd = _case(n, k, cfg)
        y_ws = w4.w4a16_gemv(pq, ps, xd, n, k)
        y_na = torch.full((n,), float("nan"), dtype=torch.float16, device="cuda")
        L.w4a16_gemv_noalloc(pq, ps, xd, y_na, n, k)
        torch.cuda.synchronize()
        assert torch.equal(y_ws.view(torch.int16), y_na.view(torch.int16)), (n, k)
        # a second call on the shared array (left zero by the first) agrees too
        y2 = torch.zeros_like(y_na)
        L.w4a16_gemv_noalloc(pq, ps, xd, y2, n, k)
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), y_na.view(torch.int16)), (n, k)
        assert_gemv(y_na.cpu().numpy().astype(np.float64), oracle.gemv(q, s, x), f"noalloc {n}x{k}")


def test_noalloc_gemv_refuses_shapes_beyond_its_workspace():
    lib = w4.lib()
    cap = lib.w4_noalloc_scratch_bytes()
    assert cap == 4 << 20
    # a matrix of 1 << 22 rows needs more than the fixed workspace
    assert lib.w4_gemv_ws_bytes(1 << 22, 128) > cap
    dummy = torch.zeros(64, dtype=torch.int16, device="cuda")
    p = dummy.data_ptr()
    assert lib.w4a16_gemv_noalloc(p, p, p, p, 1 << 22, 128, None) == L.W4_EINVAL
    assert lib.w4a16_gemv_noalloc(p, p, p, p, 64, 100, None) == L.W4_EINVAL
