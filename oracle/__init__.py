"""CPU oracle for the fused FP8 MoE layer (one GPU's expert-parallel share).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its Python binding)
never imports, calls or links it, and it shares no code with that path.

The oracle is plain, slow and written to be checked by eye against the pages:

  * "Mega-MoE notes, part 2: index table and pull" (kwkr.cn) -- index-table coordinates
    (section 1), expert segmentation of the pool (2.4), round-robin source choice (2.5),
    the per-row pull (2.6), per-128-K scale promotion (5.2).
  * "Mega-MoE kernel code walkthrough: from Dispatch to WGMMA" (mlqm.cn) -- expert to rank
    map (section 2), top-k lane walk and counting (4.1, 4.2), table write (4.3), the two
    FFN layers and their epilogues (section 6), scale promotion (8.1).
  * "DeepGEMM Mega MoE symmetric memory deep analysis" (backyes deepepv2, ch. 09) -- buffer
    layout and pool capacity (4.1, 4.2), min-peeling round-robin (7.5), scatter of the
    second layer into the per-top-k combine buffer (8.1, 8.2), top-k reduce (9.2),
    gate/up halves of W1 (10.2).
  * "Dispatch/Combine: blog theory vs DeepEP vs DeepGEMM Mega MoE" (backyes deepepv2,
    06_01) -- the combine identity (section 1), counting sort (4.4), expert-major pool
    with BLOCK_M padding (5.3), TokenSrcMetadata (6.2).
  * "MoE fused operators" (mkbk-pku.cn) -- pull, then L1 GEMM + SwiGLU, then L2 GEMM +
    scatter, then weighted reduce (DeepGEMM MegaMoE part, sections 0-5).

Precision: fp64 throughout, except where the pages fix a precision or a floating-point
value decides an integer: the FP8 requantisation decision is taken in fp32 (the kernel's
precision), the second layer's output is stored as bf16 in the combine buffer (as the
pages' L2 epilogue does) and the layer output is bf16.

Every function is pinned by the CPU tests (tests/test_oracle_*.py) against worked examples
printed on the pages, closed forms, invariants, library routines and brute force.
"""
from .fp8 import (e4m3fn_decode, e4m3fn_encode, bf16_round, bf16_bits)  # noqa: F401
from .fp4 import (e2m1_decode, e8m0_decode, unpack_fp4, dequant_mx)  # noqa: F401
from .layer import (route, pool_offsets, rr_inverse, rr_position, rr_sequence,  # noqa: F401
                    fill_pool, dequant_rows, dequant_blocks, expert_ffn_rows, expert_ffn_rows_bf16, swiglu,
                    requant_rows, forward, direct_token, ffn_dequantised, dequant_weight, RouteResult)
