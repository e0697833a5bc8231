"""CPU oracle (float64, numpy) for the routed-expert quantized MoE path.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (bf16_to_f64, f16_to_f64, unpack_u4, unpack_u2, unpack_u1,  # noqa: F401
                         dequant_int4, dequant_mwq, dequant_delta2, mwq_code, route_topk,
                         permute, silu, round_bf16, swiglu_expert, unpermute_combine, moe_forward,
                         delta_linear, compare)
