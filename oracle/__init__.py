"""Plain CPU oracle for batch-1 MoE decode with MXFP4 experts and an FP8 LM head.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
HIP library never calls it, and it never calls the HIP library: the two share no
code.  Inputs for both sides come from the separate ``synth`` package, which
holds no arithmetic of the method.

Everything here is written for a reader to check by eye against the sources:
numpy in float64 (float32 only where a float32 operation decides an integer
code, and then exactly the float32 operation that decides it), no blocking, no
fusion, no reordering beyond the definitions.

Sources cited in this package
  [news]  yoususu.cn/post/959 -- news article on NVIDIA's software-only DGX Spark
          decode speed-up (sections: "where the speed comes from", "real
          workloads", "two easily missed details", "boundary").
  [ic]    ic.work article on DGX Spark running Ling-3.0-flash (sections: "three
          scalpels" on the 5.1B-active / 157K-vocab model, "hardware").
  [card]  ai.cheesepanini.fun knowledge card "three ways to boost MoE inference
          on DGX Spark" (sections: summary, background, method points #1-#3,
          results, why it matters, limits).
  [MX]    OCP Microscaling Formats (MX) Specification v1.0 (E2M1 element,
          E8M0 shared scale, 32-element blocks).
  [OFP8]  OCP 8-bit Floating Point Specification (OFP8) rev 1.0 (E4M3 encoding).

Parity status of each function is listed in the module that defines it.
"""

from .formats import (
    e2m1_value,
    e8m0_value,
    mxfp4_dequant,
    e4m3_value,
    e4m3_encode_rne_sat,
    bf16_round,
    bf16_bits,
)
from .route import route_topk, dispatch_table, router_logits, expert_groups
from .moe import expert_ffn, moe_layer, moe_layer_by_expert, rmsnorm
from .lmhead import (lmhead_quant_fp8, lmhead_gemv_fp8, lmhead_gemv_fp8_dynact, lmhead_gemv_bf16, lmhead_argmax,
                     lmhead_sample)

__all__ = [
    "e2m1_value", "e8m0_value", "mxfp4_dequant", "e4m3_value",
    "e4m3_encode_rne_sat", "bf16_round", "bf16_bits",
    "route_topk", "dispatch_table", "router_logits", "expert_groups",
    "expert_ffn", "moe_layer", "moe_layer_by_expert", "rmsnorm",
    "lmhead_quant_fp8", "lmhead_gemv_fp8", "lmhead_gemv_fp8_dynact", "lmhead_gemv_bf16", "lmhead_argmax",
    "lmhead_sample",
]
from .shared_fp8 import quant_fp8_rows, dequant_fp8_rows, shared_fp8_dense
