// Internal declarations shared by the library's translation units.
#pragma once
#include <cstddef>
#include <cstdint>

namespace svdq {

// Shape rules common to every entry point (see svdq.h).
int validate_shape(int K, int N, int rank, int group);

// Compute units of the current device, looked up once per device (256 when
// the runtime cannot tell); safe to call from several host threads.
int device_cu_count();
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
// One row (M = 1, K <= 8192), activation scaling fused in: y = the two
// kernels' output from x and inv_scale directly.
int launch_awq_linear_row(const void* x, const float* inv_scale, const void* w_codes, const void* w_scales,
                          const void* w_zeros, const void* bias, int N, int K, void* y, void* stream);

// svdq_fp6_kernels.hip (kernel 1's FP6 mode is in svdq_kernels.hip)
int launch_quant_act_lora_down_fp6(const void* x, const float* smooth_inv, const void* lora_down, int M, int K,
                                   int rank, int act, void* x_fp6, void* x_scales, float* lora_act, void* stream);
int launch_gemm_w4a4_fp6(const void* x_fp6, const void* x_scales, const void* w_fp6, const void* w_scales,
                         const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K, int rank,
                         int out_dtype, void* y, void* stream);
// 256 x 192 tiles in the transposed form (svdq_fp6_n192_kernels.hip); w_fp6
// in the plain fragment layout, N % 192 == 0.
int launch_gemm_w4a4_fp6_n192(const void* x_fp6, const void* x_scales, const void* w_fp6, const void* w_scales,
                              const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K,
                              int rank, int out_dtype, void* y, void* stream);
// 1 when the 256 x 192 form is expected to be faster for this M and N.
int fp6_n192_preferred(int M, int N);
// The kernels an INT4 layer expected to be fastest for an M x N output: 0 the
// 6-bit kernel 2 in 256 x 256 tiles, 1 in 256 x 192 tiles, 2 the int8 engine.
int fp6_route(int M, int N);
// The same kernel with the fused QKV epilogue (one tile per block).
int launch_gemm_w4a4_fp6_qkv(const void* x_fp6, const void* x_scales, const void* w_fp6, const void* w_scales,
                             const float* lora_act, const void* lora_up, const void* bias, const void* norm_q,
                             const void* norm_k, const float* rope_cos, const float* rope_sin, float eps, int M, int N,
                             int K, int rank, int out_dtype, void* y, void* stream);

// The MLP chain (svdq_fp6_kernels.hip): kernel 2 of the up layer with the
// down layer's kernel-1 work in its epilogue, then the partials' reduction.
int launch_mlp_chain_fp6(const void* x_fp6, const void* x_scales, const void* w_fp6, const void* w_scales,
                         const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K, int rank,
                         const float* smooth_inv_dn, const void* lora_down_dn, int rank_dn, void* x_fp6_dn,
                         void* x_scales_dn, float* lora_act_dn, float* partials, void* stream);

// The chain's device-resident scratch for the no-allocation entry point:
// its size, and the current device's address (looked up once per device).
size_t chain_scratch_bytes();
int chain_scratch(void** ptr);

// svdq_probes.hip
int launch_probe_mfma(int kind, int blocks, int iters, void* sink, void* stream);
double probe_mfma_ops(int kind, int blocks, int iters);
}  // namespace svdq
