"""Plain, slow CPU oracle of the deflated ASP NVFP4 W4A4 linear layer.

TEST INFRASTRUCTURE ONLY. Nothing in the library (``wam_asp_w4a4_amd``) imports,
calls or links anything here; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP path:
it is written in NumPy, in float64, from the method's statement on these pages:

* "FastWAM UR3 3-task -- 4-bit quantisations" (Hugging Face model card), section
  "What ASP is, and what the deflated form means" (the deflated contract), the
  method table at the top (NVFP4 = E2M1 elements, block 16, E4M3 block scales,
  W4A4 with both operands at block 16) and section "Verification -- NVFP4
  deflated ASP" (bf16 output cast, no dequantised weight copy).
* "Q-WAM: 4-Bit Quantization of World Action Models with Action-Subspace
  Protection" (abstract): the protected directions live in a 16-bit low-rank
  branch; the complement of weights and activations is quantised to 4 bits.

Modules:
  formats  -- E2M1 / E4M3FN codecs (round-to-nearest-even, saturating) and the
              NVFP4 block quantiser / dequantiser.
  hadamard -- Sylvester Hadamard matrices and the block Hadamard rotation.
  asp      -- fp64/fp32/bf16 rounding helpers, the weight side (pack; the
              deflated and the shared-weight arm), the activation side and the
              layer forward.
  smoothing -- the per-layer (alpha, beta) smoothing search.
  eigen    -- the top-r eigenspace of a symmetric PSD metric (the basis V).
  svdquant -- the SVDQuant-style INT4 (group 64) W4A4 layer: quantiser, rank-r
              16-bit branch, residual, forward.

Every function here is pinned by tests under ``tests/test_oracle_*.py`` against
closed forms, hand-derived vectors (``tests/golden/``), invariants and brute force.
"""

from . import formats, hadamard, asp, smoothing, eigen, svdquant  # noqa: F401
