"""CPU oracle for the W4A16 skinny GEMM and the top-8 MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, tables or helpers); the two meet only
in the seeded inputs that ``synth`` draws.

Everything is plain NumPy in float64.  Each function states the passage of
the pages it follows and how it is pinned (see ``tests/test_oracle_*.py``).

Pages cited:
  [README]  gemma-cuda-hybrid README -- "Everything it has", "Why it's
            NVIDIA-only" (NVFP4 W4A16: E2M1 codes, E4M3 group-16 scales,
            fp32 global scale; M <= 16 GEMMs; grouped MoE top-8 + 1 shared).
  [ISSUE]   TensorFold issue "Proposal: Gemma 4 on CUDA" -- "Why now"
            (qlinear's MLX affine paths in groups of 64, activation rows with
            64-value group sums, tree_round's argmax), "Gates" (float64 bound).
  [DOC]     TensorSharp docs, Gemma 4 -- section 3.2 "Per-layer (MoE)",
            4.6 "MoE" (router matmul, softmax, top-k, weighted sum of
            experts), 4.8 "Logit softcap", 14 "Completed: Expert-batched
            FFN (GEGLU)".
"""
from .formats import (e2m1_value, e4m3_value, unpack_nibbles, nvfp4_dequant,
                      nvfp4_dequant_f32, bf16_value, affine_dequant, affine_dequant_f32,
                      affine_dequant_bits, AFFINE_BITS)
from .gemm import (gemm_ref, gemm_abs_bound, nvfp4_gemm_ref, affine_gemm_ref,
                   affine_gemm_groupsum, argmax_ref, affine_bits_gemm_ref)
from .moe import (gelu_tanh, gelu_tanh_deriv, softmax, route_topk, moe_ref,
                  moe_ref_grouped, moe_abs_bound, a16)
from .sampling import (philox4, uniform_bits_to_f32, sample_uniforms, gumbel, softcap,
                       sample_scores, sample_tokens)
from .block import (rmsnorm, rmsnorm_bound, route_normed, route_normed_bound, routing_weight_bound,
                    moe_block_ref, moe_block_bound)
from .quantize import e4m3_encode_rne, e2m1_encode_rne, nvfp4_global_scale_f32, nvfp4_quantize_f32

__all__ = [
    "e2m1_value", "e4m3_value", "unpack_nibbles", "nvfp4_dequant", "nvfp4_dequant_f32",
    "bf16_value", "affine_dequant", "affine_dequant_f32", "gemm_ref", "gemm_abs_bound",
    "nvfp4_gemm_ref", "affine_gemm_ref", "affine_gemm_groupsum", "argmax_ref",
    "gelu_tanh", "gelu_tanh_deriv", "softmax", "route_topk", "moe_ref", "moe_ref_grouped",
    "moe_abs_bound", "a16", "philox4", "uniform_bits_to_f32", "sample_uniforms", "gumbel", "softcap",
    "sample_scores", "sample_tokens", "e4m3_encode_rne", "e2m1_encode_rne", "nvfp4_global_scale_f32", "affine_dequant_bits", "AFFINE_BITS", "affine_bits_gemm_ref",
    "rmsnorm", "rmsnorm_bound", "route_normed", "route_normed_bound", "routing_weight_bound", "moe_block_ref",
    "moe_block_bound",
    "nvfp4_quantize_f32",
]
