"""CPU oracle for the ternary (BitNet b1.58) and sign-only (OneBit) linear layers.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The HIP library never calls it and
shares no code with it; the two meet only through the seeded inputs of
``synth``.

Everything here is deliberately plain: NumPy in fp64 / int64 (or fp32 exactly
where a quantised integer is decided in fp32, as the kernels do), one step per
definition, no blocking or fusion. Sources, cited by page title and section:

* [b158] "微软、国科大开启1Bit时代：大模型转三进制，速度快4倍能耗降至1/41"
  (BitNet b1.58 write-up), sections "BitNet b1.58 介绍" and "实验及结果".
* [onebit] "清华、哈工大把大模型压缩到了1bit，把大模型放在手机里跑的愿望就快要实现了！"
  (OneBit write-up), section "OneBit 框架" (1. new 1-bit structure, Fig. 3;
  2. SVID; 3. knowledge distillation) and "讨论与分析 / 1. 效率".
* [billm] "BiLLM: Pushing the Limit of Post-Training Quantization for LLMs"
  blog summary, sections "方法细节" (step 2, residual approximation) and
  "存储位开销分析".

Readings taken where the pages are silent are stated in each function. Parity status
of each function is in its docstring.
"""
from .formats import (pack_ternary, unpack_ternary, pack_ternary_mf, unpack_ternary_mf,
                      pack_sign, unpack_sign, act_planes, ternary_packed_bytes,
                      sign_packed_bytes)
from .b158 import (QB, exact_abs_sum, f32_nearest, absmean_beta, ternarize_absmean,
                   quant_act_int8, acc_exact, bitlinear_output, bitlinear_forward)
from .onebit import (onebit_forward, onebit_error_scale, onebit_storage_bits,
                     onebit_param_count, svid_rank1)
from .billm import (residual_binarize, residual_forward, residual_error_scale,
                    group_abs_mean_f32, exact_group_abs_sums, f32_nearest_dyadic,
                    billm_storage_bits_per_param)

__all__ = [
    "pack_ternary", "unpack_ternary", "pack_sign", "unpack_sign", "act_planes",
    "ternary_packed_bytes", "sign_packed_bytes",
    "QB", "exact_abs_sum", "f32_nearest", "absmean_beta", "ternarize_absmean",
    "quant_act_int8", "acc_exact", "bitlinear_output", "bitlinear_forward",
    "onebit_forward", "onebit_error_scale", "onebit_storage_bits", "onebit_param_count",
    "svid_rank1", "residual_binarize", "residual_forward", "residual_error_scale",
    "group_abs_mean_f32", "exact_group_abs_sums", "f32_nearest_dyadic",
    "billm_storage_bits_per_param",
]
