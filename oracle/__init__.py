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
* ``decode_step`` / ``forward_teacher_forced``: zero-weight special case against a
  single matmul, and sequential == batched on a tiny model — pinned;
* logits of the full 28-layer random model: parity unpinned beyond the
  component pins above (no external value exists for a random-init model).
"""
from .ref import *  # noqa: F401,F403
