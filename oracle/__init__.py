"""CPU oracle of the routed-MoE block (test infrastructure only).

A plain, slow, obviously correct numpy implementation of what the block
computes, written from the pages' statement of it.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
(the HIP library and its Python binding) never does.  It shares no code with
the HIP path.

Every function cites the passage it follows, by page title and section.
Page titles used in citations:

* [mono.decoder] vllm.models.muse_spark.amd.mono.decoder (the MI355X decode
  monokernel driver)
* [muse_moe_runner] vllm.models.muse_spark.amd.muse_moe_runner (the ROCm MoE
  runner, including the router of common/moe.py it renders)
* [mono] vllm.models.muse_spark.amd.mono (the monokernel package)
* [providers] vllm.models.muse_spark.nvidia.specialized_decode.runtime.providers

Precision: values the pages fix keep the pages' precision (fp32 router
logits, scores, selection keys and route weights; bf16 pooler output,
activations, MoE output, unpooler output and next-layer input; fp32 residual
stream).  Everything else is computed in fp64.
"""

from .steps import (  # noqa: F401
    BlockResult,
    attn_boundary,
    Routing,
    bf16_to_f64,
    block,
    boundary,
    decode_e2m1,
    decode_e8m0,
    dequant_mxfp4,
    effective_norm_weight,
    experts,
    experts_down,
    fake_quant_mxfp4,
    group_routes,
    next_qkv,
    pool,
    quantize_mxfp4,
    rms_norm,
    round_bf16,
    route,
    route_from_logits,
    router_logits,
    score,
    select_topk,
    route_weights,
    unpool,
)
