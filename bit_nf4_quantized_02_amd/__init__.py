"""QLoRA NF4 linear for MI355X (gfx950).

``bit_nf4_quantized_02_amd.qlora`` is the thin ctypes binding over the C-ABI
library ``libqlora.so`` (HIP kernels + host API, built from ``csrc/``);
``bit_nf4_quantized_02_amd.synth`` draws the seeded synthetic inputs.
Importing this package loads nothing; importing ``qlora`` loads the library
and raises if it has not been built.
"""
