// Internal declarations shared by the library's translation units.
#pragma once
#include <cstdint>

namespace svdq {

// Shape rules common to every entry point (see svdq.h).
int validate_shape(int K, int N, int rank, int group);
// Shape rules of the MXFP4 entry points (K a multiple of 128).
int validate_shape_mx(int K, int N, int rank);

// Kernel launchers (svdq_kernels.hip).  Arguments already validated.
int launch_quant_act_lora_down(const void* x, const float* smooth_inv, const void* lora_down, int M,
                               int K, int rank, int act, void* x_codes, void* x_scales,
                               float* lora_act, void* stream);
int launch_lora_down(const void* x, const float* smooth_inv, const void* lora_down, int M, int K, int rank,
                     int act, float* lora_act, void* stream);
int launch_lora_up_add(const float* lora_act, const void* lora_up, int M, int N, int rank, void* y, void* stream);
int launch_gemm_w4a4_lora_up(const void* x_codes, const void* x_scales, const void* w_codes,
                             const void* w_scales, const float* lora_act, const void* lora_up,
                             const void* bias, int M, int N, int K, int rank, int out_dtype, void* y,
                             void* stream);

int launch_gemm_w4a4_lora_up_qkv(const void* x_codes, const void* x_scales, const void* w_codes,
                                 const void* w_scales, const float* lora_act, const void* lora_up,
                                 const void* bias, const void* norm_q, const void* norm_k, const float* rope_cos,
                                 const float* rope_sin, float eps, int M, int N, int K, int rank, int out_dtype,
                                 void* y, void* stream);
int launch_quant_act_lora_down_mxfp4(const void* x, const float* smooth_inv, const void* lora_down, int M,
                                     int K, int rank, int act, void* x_codes, void* x_scales,
                                     float* lora_act, void* stream);
// svdq_mx_kernels.hip
int launch_gemm_mxfp4_lora_up(const void* x_codes, const void* x_scales, const void* w_codes,
                              const void* w_scales, const float* lora_act, const void* lora_up,
                              const void* bias, int M, int N, int K, int rank, int out_dtype, void* y,
                              void* stream);

// svdq_awq_kernels.hip
int launch_awq_quant_act(const void* x, const float* inv_scale, int M, int K, void* x_hat, float* xsum,
                         void* stream);
int launch_awq_gemv(const void* x_hat, const float* xsum, const void* w_codes, const void* w_scales,
                    const void* w_zeros, const void* bias, int M, int N, int K, void* y, void* stream);

// svdq_probes.hip
int launch_probe_mfma(int kind, int blocks, int iters, void* sink, void* stream);
double probe_mfma_ops(int kind, int blocks, int iters);
}  // namespace svdq
