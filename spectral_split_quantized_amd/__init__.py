"""MI355X-native (gfx950) Metis spectral-split NVFP4 GEMM.

The compute path is the C-ABI library ``libmetis.so`` built from the HIP
sources under ``csrc/``; ``metis`` is its thin ctypes binding.  ``synth``
makes seeded synthetic inputs.  The library is loaded on first use, and a
missing library is an error (there is no fallback path).
"""

__all__ = ["metis", "synth"]
