"""CPU oracle of the routed-expert FP8 block-scaled MoE decode step.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, calls or links
this package; only the tests, the smoke check and the benchmark's CPU
baseline do. It is a plain, slow, float64 NumPy statement of what the path
computes, written from the pages' definitions, and shares no code with the
HIP library (no kernels, headers, tables or helpers).

Pages cited (all vLLM API docs unless noted):
  * "mega_moe" page (glm5next specialized_decode): MegaExperts, top_k_pick,
    the epilogue's activation quantisation and scale-sum, hidden_block.
  * "shared_expert" page (glm5next specialized_decode): SharedExpert,
    _group_scale, _GateUpKernel, _DownKernel, block_scales.
  * "nvfp4-megamoe-kernel" README (blame view): slot representation and the
    bugs list (per-slot SiLU, routing weights applied once).
  * "kimi_k3 ... ep.comm" page: the combine's FP32 sum rounded once; the
    boundary steps of its dispatch and combine (MXFP8 quantisation of the
    latent, reduce + RMSNorm), in oracle/boundary.py.

Parity status of each function is listed in its docstring; every function
here is pinned by a `-m "not gpu"` test in tests/test_oracle_*.py.
"""

from . import boundary, fp4  # noqa: F401
from .codecs import bf16_round, e4m3_decode, e4m3_encode, f32, E4M3_VALUES  # noqa: F401
from .moe import (  # noqa: F401
    block_scaled_gemm,
    combine,
    moe_decode,
    quantize_blocks,
    requantize_hidden,
    route,
    shared_expert,
    silu_f32,
    swiglu,
    ue8m0_round_up,
    unpack_ue8m0,
)
