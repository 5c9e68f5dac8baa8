"""Fused-dequant quantized matrix-vector products (Q4_0, Q8_0, Q4_K) for
AMD Instinct MI355X (gfx950).

The compute lives in ``libqmv.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/qmv.h``).  ``quantized_dequant_matrix_amd.qmv`` is the
thin Python binding over it; ``quantized_dequant_matrix_amd.synth`` draws the
seeded synthetic inputs.
"""
__all__ = ["qmv", "synth"]
