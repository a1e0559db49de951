"""QPN weight-streaming skinny GEMM for MI355X (gfx950).

NVFP4 / FP8 weights stay compressed in HBM and are expanded in registers
inside hand-written HIP kernels; the work sits behind the C-ABI library
``libqpn.so`` (declared in include/qpn.h).  This package holds the HIP
sources (csrc/), the build step, a thin ctypes binding (``qpn``) and the
seeded synthetic input generators (``synth``).

Importing the package loads nothing; ``from fp8_quantized_skinny_qpn_amd
import qpn`` loads the library and fails loudly when it is not built.
"""
