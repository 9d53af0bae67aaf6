"""fp64 CPU oracle for the chunked gated delta rule forward pass and its decode step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
anything in this package: only the tests, the smoke check of the graft entry point
and the CPU-baseline leg of the benchmark use it. It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing); both sides
are fed from the seeded generators in ``workloads.py``, which hold none of the
method's arithmetic.

Functions (all float64 numpy):

* ``recurrent_fwd``  - the definition: the per-token gated delta rule.
* ``chunked_fwd``    - the chunked WY algorithm (recompute_w_u, chunk_fwd_h,
  chunk_fwd_o with chunk size 64), exposing its intermediates.
* ``*_varlen``       - the same over a packed token stream with sequence offsets.
* ``decode_step``    - one recurrent step over a slot-indexed state pool.
* ``decode_verify``  - T tokens per request (speculative verify) over that pool,
  with per-token state writes.
* ``recurrent_fwd_kda`` / ``decode_step_kda`` - the rule with a decay per key
  channel (KdaSplit), per token and as a decode step over the pool.
* ``decode_prologue`` / ``gated_rmsnorm`` - the decode layer's front (conv1d
  over a conv-state pool, SiLU, q/k L2 norm, sigmoid beta) and back (gated
  RMSNorm) operations (``oracle/layer.py``); ``decode_prologue_verify`` the front
  for T tokens per request with the speculative-verify conv page.
* ``kda_gate``       - the per-key-channel decays of the KDA decode layer from its
  low-rank gate projection (``oracle/gate.py``), in each of the page's float32
  reduction orders, exactly.
* ``fp8_quant``      - group quantisation to FP8 E4M3 (``oracle/fp8.py``), with
  ``e4m3_encode`` / ``e4m3_decode``.

Every function is pinned by tests in ``tests/test_oracle_pins.py`` against closed
forms, invariants and a hand-derived golden example; no function is "parity
unpinned".
"""

from .gdn import (  # noqa: F401
    recurrent_fwd,
    chunked_fwd,
    recurrent_fwd_varlen,
    chunked_fwd_varlen,
    decode_step,
    decode_verify,
    decode_step_kda,
    recurrent_fwd_kda,
    unit_lower_inverse,
)
from .fp8 import e4m3_decode, e4m3_encode, fp8_quant  # noqa: F401
from .layer import conv_silu_step, decode_prologue, decode_prologue_verify, gated_rmsnorm  # noqa: F401
from .gate import kda_gate  # noqa: F401
