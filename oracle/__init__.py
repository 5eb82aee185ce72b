"""CPU oracle for curvature-aware NVFP4 weight quantization (GPTQ + Schur Replay).

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously-correct
reference that the GPU library is checked against.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path never calls into it and shares no code with it.

Method source: "Replay the Curvature: Accurate and Scalable NVFP4 Quantization
for Large Language Model Inference" (arXiv 2609.36654), Abstract.  The abstract
fixes: NVFP4 blocks of 16 E2M1 weights sharing one E4M3 scale; the GPTQ column
sweep in which quantizing a column updates the columns that follow; Schur
Replay, which scores each candidate block scale by reproducing the GPTQ updates
that the scale causes inside the block and measuring the block error left after
compensation from the still-unquantized columns.

Arithmetic is fp64 unless a function says otherwise.  Every function cites the
passage it follows.  Readings where the pages are silent are documented at the
function that takes them.

Parity status: every function here is pinned by a CPU test (codebook and
library codecs, closed forms, brute-force least squares, invariants); see the
module docstrings.
"""

from . import codec, gptq  # noqa: F401
