"""CPU oracle for the W4A16 batch-1 decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library and never reads packed bytes: it consumes the raw
(codes, scales) arrays the ``synth`` generators produce.

Everything is plain numpy in float64, with fp16 rounding applied only at the
storage points the method defines (see ``oracle.ref``).  Pins that tie it to
something other than itself live in ``tests/test_oracle_pins.py``.

Parity status of each function (what pins it):

* ``deq``, ``gemv``: exhaustive exactness + rational brute force — pinned;
* ``quantize_int4`` (fp16 -> int4 weights): exact-rational brute force of its
  definition, reconstruction bound, extremes and zero groups — pinned;
* ``quantize_act_int8``, ``gemv_w4a8`` (int8 activations): rational brute force of
  the quantiser's definition, reconstruction bound, extreme-value and zero-group
  cases, exact rational GEMV, and equality with ``gemv`` when the activations
  are exactly representable — pinned;
* ``rmsnorm``, ``rope``, ``silu``, ``swiglu``: closed forms and invariants — pinned;
* ``paged_attention``, ``causal_attention``: one-token, two-token closed form,
  uniform-key mean, GQA mapping, page-shuffle invariance — pinned;
* ``mlp``: identity and scaled-identity projections with a closed-form result —
  pinned;
* ``layer_step`` / ``decode_step`` / ``forward_teacher_forced``: a hand-built
  one-layer model whose every intermediate has a closed form (distinct ln1, ln2
  and final-norm weights, bias before RoPE at two positions, the QKV split
  order, the MLP fed the second norm, both residual adds), planted wiring
  mistakes that must fail it (``tests/test_oracle_layer_pins.py``,
  ``tests/test_oracle_mutants.py``), the zero-weight special case against a
  single matmul, and sequential == batched on a tiny model — pinned;
* ``act_int8`` and the ``act="int8"`` step mode: equal to ``quantize_act_int8``
  dequantised, the layer's four quantised GEMV inputs checked against
  ``gemv_w4a8`` with planted mistakes, sequential == batched
  (``tests/test_oracle_int8_mode.py``) — pinned;
* logits of the full 28-layer random model: parity unpinned beyond the
  component pins above (no external value exists for a random-init model).
"""
from .ref import *  # noqa: F401,F403
