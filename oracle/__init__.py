"""CPU oracle for the QLoRA NF4 linear — TEST INFRASTRUCTURE ONLY.

This package is the slow, plainly written reference that the HIP library is
checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product library and its
Python binding never do, and nothing here imports them. It shares no code,
table or constant generator with the HIP path: the codebook, the FP8 table,
every rounding step and both GEMM formulas are written out again here from the
pages' description of the method.

Modules
-------
``oracle.nf4``     codebook, blockwise NF4 quantization, double quantization of
                   the block constants, dequantization to bf16; the uniform
                   INT4 grid and the encoding without double quantization
                   (ablations).
``oracle.linear``  fp64 forward and backward of the frozen-base linear with the
                   LoRA branch, plain and with dropout on the branch's input,
                   and the element-wise error bound of an fp32-accumulated
                   16-bit result.
``oracle.merge``   the adapter folded into a dequantized copy of the base (and
                   taken out again), exact in fp64, rounded once.
``oracle.adamw``   the AdamW step on the adapter and its learning-rate schedule.
``oracle.mlp``     the gated-MLP join silu(G) * U and its gradients, which chains
                   the MLP linears of the 7B block and the 65B-class stack.

Every function is pinned by ``tests/test_oracle_*.py`` against facts that do
not come from this code (values the pages print, closed forms, brute force,
library routines for special cases). No function here is "parity unpinned".
"""

from . import nf4, linear, merge, adamw, mlp  # noqa: F401
