"""MI355X (gfx950) W4A16 batch-1 decode path.

Python side of libw4a16.so: argument marshalling over the C ABI declared in
``include/w4a16.h``.  The entry points keep the library's names:
``pack_int4_weights``, ``w4a16_gemv``, ``paged_attn_decode``, ``decode_step``,
for prompt prefill ``w4a16_gemm``, ``paged_attn_prefill``, ``prefill``, and for
int8 activations ``w4a8_quantize_act``, ``w4a8_gemv``.
"""
from ._lib import (W4Error, W4_EAGER, W4_GRAPH, W4_MULTI, W4_PERM_GATE_UP, W4_PERM_QKV, ModelConfig,  # noqa: F401
                   lib, model_row_perm, pack_f16_matrix, pack_int4_weights, paged_attn_decode,
                   paged_attn_prefill, quantize_int4_weights, unpack_int4_weights, w4a8_gemv, w4a8_quantize_act, w4a16_gemm,
                   w4a16_gemv, w4a16_mlp)
from .model import DecodeModel, decode_step, prefill  # noqa: F401
