"""MI355X-native MiniMax Sparse Attention (MSA) hot path.

The compute lives in ``libmsa.so`` (hand-written HIP kernels for gfx950 behind a
C ABI, declared in include/msa.h). This package holds the thin ctypes binding
(:mod:`.binding`) and the seeded input generators (:mod:`.inputs`).
"""
