"""CPU fp64 oracle for the MiniMax Sparse Attention (MSA) hot path.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously-correct
reference that the HIP library is checked against.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
path (the C-ABI library and its Python binding) never does, and there is no
CPU fallback that routes through it.

It shares no code, tables or constants with the HIP library.  Every function
cites the passage of the source pages it follows:

* "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援" (the English post on
  hot.atechcom.net), sections "MSA primer", "What is new in the MiniMax-M3.1
  architecture", "NVIDIA Blackwell optimized MSA kernels", "NVIDIA Rubin
  optimized MSA" and "NVFP4 MSA kernel" (AMD).

Modules:
  formats  -- E2M1 / E4M3 decoding, RNE encoders, NVFP4 and FP8 quantisers and
              the two NVFP4 dequantisation readings (exact, FP8-rounded).
  msa      -- indexer scores, block max-pool, top-16 selection with the own
              block forced, exact sparse attention, and the whole layer step.
  traffic  -- the algorithmic bytes / FLOP model of one layer step.

Parity status of each function is stated in its docstring; every function
here is pinned by a ``-m "not gpu"`` test against something other than itself.
"""
from . import formats, msa, traffic  # noqa: F401
