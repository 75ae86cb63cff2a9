"""CPU oracle for block-scaled quantization of MoE token rows.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously-correct
reference that the HIP path is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code, tables or constants with the HIP library and
the library never imports it.

Source pages (cited by title and section):

* P1 -- "[Common][PyTorch] Add NVFP4 EP dispatch and combine backward"
  (TransformerEngine PR #3753): PR description and commit messages.
* P2 -- "[Common][PyTorch] EP dispatch with unfused MXFP8 quantization"
  (TransformerEngine PR #3270): description, "Changes", review comments.
* P3 -- "[PyTorch] Enable NVFP4 row-scaled (per-token) backward for
  GroupedLinear" (TransformerEngine PR #3324): description, bot summary.
* P4 -- "[PyTorch] Optionally derive FC1 dy NVFP4 amaxes from the dGLU
  epilogue" (TransformerEngine PR #3755): description, test commit.

The pages name the formats and the passes but fix no rounding rule, constant,
byte order or random-number mapping.  Every such rule is a reading written out
in the docstring of the function that implements it (rules R1..R21, R8b: a
second stochastic-rounding decision rule, the carry form, and R22..R23 in
``mxfp4``: an MXFP4 variant of the receive that no page describes).

Precision: where a rule says ``fl32(.)`` the oracle computes in numpy float32
(IEEE binary32, round-to-nearest-even, gradual underflow); everything else is
exact (float64 on values that float64 holds exactly, or integer arithmetic).

Parity status: every function is pinned by a CPU test in ``tests/`` against
something other than itself, except the choice of the RHT sign vector (an
arbitrary fixed constant by design) -- parity unpinned for that choice only.
"""

from . import formats, philox, nvfp4, mxfp8, mxfp4, routing, rht, receive, dswiglu  # noqa: F401
