"""SmoothQuant W8A8 quantized linear for MI355X (gfx950).

The compute lives in ``libsq.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/sq.h``). ``binding`` marshals torch tensors into that
ABI; ``inputs`` draws the seeded synthetic workloads.
"""
__all__ = ["binding", "inputs"]
