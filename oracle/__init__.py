"""Plain float64 CPU oracle for the Metis spectral-split NVFP4 GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code, tables or constants generators
with the HIP library under ``spectral_split_quantized_amd/``; the only thing
both sides consume in common are the seeded inputs made by
``spectral_split_quantized_amd.synth`` (which holds none of the method's
arithmetic).

Sources.  The method is described on the web page "Metis: Training LLMs with
FP4 Quantization" (ICLR 2026 reading notes): section 关键设计 1 (spectral split
M = U_k S_k V_k^T + M_R and the split forward GEMM equation for Y-hat),
关键设计 2 (sparse row sampling and Gaussian random projection), 关键设计 3
(factor reuse across steps), 研究背景与动机 (NVFP4: E2M1 values, blocks of 16,
one FP8 scale per block) and 损失函数/训练策略 (W4A4G4, stochastic rounding,
rank 1.5%, refresh every 8 steps).  Where the pages are silent the modules
state the reading they take.

Modules
-------
philox     Philox4x32-10 counter-based generator (Salmon et al., SC'11).
formats    E2M1 / E4M3 encode and decode, bit-exact.
nvfp4      the NVFP4 fake quantiser (RNE and stochastic rounding) + dequant.
linalg     cyclic Jacobi eigensolver, one-sided Jacobi SVD, shifted CholeskyQR3.
rsvd       Omega table, row sampler, randomized sketch, projection/rediag,
           residual and the factor cache.
split_gemm dense-dequant reference of the split forward and backward GEMMs.

Parity status: every function is pinned by ``tests/test_oracle_*.py`` except
the exact Philox output stream, which is "parity unpinned" (no published
known-answer vectors are available here; only its published constants and its
statistics are checked).
"""

from . import philox, formats, nvfp4, linalg, rsvd, split_gemm  # noqa: F401
