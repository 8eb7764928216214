"""CPU oracle for the fused MoE decode-layer step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy statement of what one decoder-layer launch computes, as
described on the LMSYS / SGLang "Muse Spark Open" megakernel pages: attention of
layer L over the KV cache for a 16-token verification tree, the output projection,
the pooler, the top-8-of-256 router, the NVFP4 expert GEMMs with SwiGLU, the
unpooler, and layer L+1's qkv projection with its KV-cache write.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the
benchmark may import this package.  It shares no code with the HIP path; the only
module both sides use is ``synth`` (seeded inputs, no layer arithmetic).
"""
from .numerics import (bf16_round, bf16_to_f64, e2m1_value, e4m3_value, e4m3_rne_scale,
                       nvfp4_pack, nvfp4_decode, fp4_act_quant, E2M1_GRID, E4M3_POS)
from .layer import (tree_masks, visible_keys, attention, dense, router, moe, silu, qkv_project,
                    layer_step, layer_step_auto, used_experts, pack_experts, usage_top)
from .accept import tree_accept, kv_commit

__all__ = ["bf16_round", "bf16_to_f64", "e2m1_value", "e4m3_value", "e4m3_rne_scale",
           "nvfp4_pack", "nvfp4_decode", "fp4_act_quant", "E2M1_GRID", "E4M3_POS",
           "tree_masks", "visible_keys", "attention", "dense", "router", "moe", "silu", "qkv_project",
           "layer_step", "layer_step_auto", "used_experts", "pack_experts", "usage_top", "tree_accept", "kv_commit"]
