"""Tiny layer shapes for the brute-force pins and quick parity cases."""
import math

from synth import CONFIGS, LayerSpec

TINY = {
    "bf16": LayerSpec(name="tiny_bf16_t", cfg_id=101, fmt="bf16", H=64, I=32,
                      n_routed=4, top_k=2, w13_std=0.1, w2_std=0.1),
    "fp8_clamp_shared": LayerSpec(name="tiny_fp8_t", cfg_id=102, fmt="fp8",
                                  H=128, I=128, n_routed=4, top_k=2, shared=1,
                                  limit=10.0),
    "fp8_oai": LayerSpec(name="tiny_fp8_oai_t", cfg_id=103, fmt="fp8", H=128,
                         I=128, n_routed=4, top_k=2, alpha=1.702, beta=1.0,
                         limit=7.0, logits="skewed"),
    "int4": LayerSpec(name="tiny_int4_t", cfg_id=104, fmt="int4", H=64, I=32,
                      n_routed=4, top_k=2),
    "ep_lora": LayerSpec(name="tiny_ep_lora_t", cfg_id=105, fmt="fp8", H=128,
                         I=128, n_routed=8, n_sink=2, top_k=3, E_loc=3,
                         offset=2, lora_rank=4, gscale=True, logits="mix258",
                         route_scale=1.5, lora_down=True),
}
# eight adapters in one batch (tokens pick one or none)
TINY["ep_lora_multi"] = TINY["ep_lora"].scaled(name="tiny_ep_lora_multi_t", cfg_id=106,
                                               n_adapters=8)
# NVFP4 weights with per-half W13 and per-expert W2 global scales, LoRA on
# both projections; MXFP4 with a shared expert
TINY["nvfp4_lora"] = LayerSpec(name="tiny_nvfp4_lora_t", cfg_id=107, fmt="nvfp4",
                               H=128, I=128, n_routed=8, n_sink=2, top_k=3, E_loc=3,
                               offset=2, lora_rank=4, gscale=True, logits="mix258",
                               route_scale=1.5, lora_down=True)
TINY["mxfp4_shared"] = LayerSpec(name="tiny_mxfp4_t", cfg_id=108, fmt="mxfp4", H=128,
                                 I=128, n_routed=4, top_k=2, shared=1, limit=7.0)
# FP8 layers with H = I = 256: each GEMM spans two 128-deep K blocks and two
# 128-row weight-scale blocks, and h spans two 128-column requant groups, so
# the blockwise grouping of the activation scales, the weight scales and the
# h re-quantisation is exercised (one group per row cannot tell per-group
# from per-row scaling)
TINY["fp8_2grp_shared"] = LayerSpec(name="tiny_fp8_2grp_t", cfg_id=109, fmt="fp8",
                                    H=256, I=256, n_routed=4, top_k=2, shared=1,
                                    limit=10.0)
TINY["ep_lora_2grp"] = LayerSpec(name="tiny_ep_lora_2grp_t", cfg_id=110, fmt="fp8",
                                 H=256, I=256, n_routed=8, n_sink=2, top_k=3, E_loc=3,
                                 offset=2, lora_rank=4, gscale=True, logits="mix258",
                                 alpha=1.702, beta=1.0, limit=7.0, lora_down=True)
# MXFP4 weights with MXFP8 activations into GEMM1, H = 256 (eight 32-column
# activation groups per row, two 128-deep K blocks), OAI SwiGLU
TINY["mxfp4a8_oai"] = LayerSpec(name="tiny_mxfp4a8_t", cfg_id=111, fmt="mxfp4_a8", H=256,
                                I=128, n_routed=4, top_k=2, shared=1, alpha=1.702,
                                beta=1.0, limit=7.0)
