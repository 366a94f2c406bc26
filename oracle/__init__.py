"""CPU oracle for the strict token-logprob path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It is a plain float64 numpy
implementation written from the definitions of the full-vocabulary
log-softmax and of the top-k/top-p sampling support, and it shares no code
with the HIP library.

Pinning: every function here is checked by ``tests/test_oracle_pins.py``
against references that do not reuse its code (50-digit mpmath sums, closed
forms, normalisation invariants, torch's float64 log_softmax, exhaustive
subset enumeration with exact rational masses, the temperature-to-zero
limit). No function in this package is parity-unpinned.
"""
from .logp import (NucleusInfo, decode_bf16, nucleus_logp, nucleus_row, ref_logp,  # noqa: F401
                   ref_logp_row, scale_fp32)
