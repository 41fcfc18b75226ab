/*
 * svdq.h -- C ABI of the SVDQuant W4A4 linear with a rank-r 16-bit branch
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer computes
 *     Y = Q4(X diag(lambda)^-1) Q4(R) + bf16(X diag(lambda)^-1 L1) L2 + bias
 * where diag(lambda) W = L1 L2 + R (W in [K x N] math layout), L1 L2 is the
 * top-r SVD of the smoothed weight and R is the 4-bit residual
 * (svdq-int4-flux.1-depth-dev model card, "Quantization Method -- SVDQuant",
 * stages 2 and 3; "Bringing Nunchaku 4-bit Diffusion Inference to
 * Diffusers", "Background: SVDQuant and Nunchaku").
 *
 * Two device entry points follow the fusion the model card's "Nunchaku
 * Engine Design" describes: the down projection runs in the same kernel as
 * the activation quantizer (both read the 16-bit input), and the up
 * projection runs in the 4-bit GEMM kernel, into the same fp32 accumulators
 * (both write the 16-bit output).
 *
 * Conventions for every function:
 *  - Return value: SVDQ_OK (0) or a negative svdq_status.  Arguments are
 *    validated on the host before anything is launched; on error nothing is
 *    written and nothing is launched.
 *  - Storage types: bf16 and fp16 values travel as their 16-bit patterns
 *    (uint16_t / void*), packed INT4 codes as bytes holding two codes each,
 *    low nibble = even k, two's complement (-8 .. 7).
 *  - Weight layouts follow torch.nn.Linear: [out_features][in_features].
 *  - The low-rank factors are stored transposed with respect to the
 *    formula above, in the same [out][in] layout as the weight:
 *    lora_down = L1^T [rank][K] (the down projection as a Linear(K -> rank))
 *    and lora_up = L2^T [N][rank] (the up projection as a Linear(rank -> N)).
 *    Kernel 1 then reads each rank row as a contiguous run along K next to
 *    the activation row it multiplies, and kernel 2 reads each output
 *    column's rank values as one contiguous run, as it reads its codes.
 *  - The library never allocates or frees memory and keeps no pointer after
 *    returning.  Device functions are asynchronous on the caller's stream,
 *    a hipStream_t passed as void* (NULL = the default stream) so that this
 *    header compiles without the HIP headers (plain C and ctypes callers);
 *    buffers must stay alive until the stream has finished.  Faults during
 *    execution surface at the caller's next synchronization.
 *  - Only group = 64 is supported.  K must be a positive multiple of 64,
 *    N a positive multiple of 8, 0 <= rank <= min(K, N), rank % 16 == 0 and
 *    rank <= SVDQ_MAX_RANK.  M >= 0 (M == 0 launches nothing).
 *  - Thread safety: no mutable global state except a per-device cache of
 *    the architecture check.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum svdq_status {
  SVDQ_OK = 0,
  SVDQ_ERR_INVALID_ARG = -1,        /* null pointer, negative or inconsistent size */
  SVDQ_ERR_UNSUPPORTED_SHAPE = -2,  /* valid request this build does not implement */
  SVDQ_ERR_UNSUPPORTED_DEVICE = -3, /* no device, or not gfx950 */
  SVDQ_ERR_HIP = -4,                /* HIP runtime call or launch failed */
  SVDQ_ERR_NUMERIC = -5             /* non-finite input, fp16 scale overflow, SVD failure */
} svdq_status;

enum { SVDQ_ACT_NONE = 0, SVDQ_ACT_GELU_TANH = 1 };
enum { SVDQ_OUT_BF16 = 0, SVDQ_OUT_F32 = 1 };
enum { SVDQ_GROUP = 64, SVDQ_MAX_RANK = 256, SVDQ_QKV_HEAD_DIM = 128, SVDQ_AWQ_MAX_ROWS = 16,
       SVDQ_AWQ_ROW_MAX_K = 8192 };

/* Human-readable name of a status code (static storage, never NULL). */
const char* svdq_status_string(int status);

/* ABI version (major * 100 + minor). */
int svdq_version(void);

/* Validates that HIP device `hip_device` exists and is a gfx950 (MI355X).
 * The pages' loader checks the GPU's capability when a quantized model is
 * loaded and refuses with a clear error rather than computing wrong results
 * ("Bringing Nunchaku 4-bit Diffusion Inference to Diffusers", "Hardware
 * support"); every device entry point below performs this check (cached per
 * device) and returns SVDQ_ERR_UNSUPPORTED_DEVICE before launching anything.
 * The environment variable SVDQ_ASSUME_ARCH, when set, replaces the queried
 * architecture name (to exercise the refusal path on any machine). */
int svdq_device_check(int hip_device);

/* Bytes of one prepared layer as produced by svdq_prepare_weights: packed
 * codes N*K/2 + fp16 scales 2*(K/64)*N + bf16 factors 2*rank*(K+N) + fp32
 * smooth_inv 4*K.  Validates the shape like the functions below. */
int svdq_prepared_bytes(int K, int N, int rank, int group, size_t* bytes_out);

/* Host, synchronous.  Offline preparation of one linear layer (stages 2 and
 * 3 of "Quantization Method -- SVDQuant" plus the 4-bit residual).
 *
 *   weight     [N][K] bf16   the layer weight (torch.nn.Linear layout)
 *   act_absmax [K]    fp32   calibration statistic max_m |X[m, k]| (>= 0)
 *   alpha             fp32   smoothing strength in (0, 1); 0.5 is the default
 *   rank, group              branch rank r and INT4 group (64)
 * Outputs (caller-owned host buffers):
 *   smooth_inv [K]       fp32  1/lambda_k with lambda_k =
 *                              max(a_k,1e-5)^alpha / max(w_k,1e-5)^(1-alpha),
 *                              w_k = max_n |weight[n][k]| (alpha = 0.5: sqrt(a/w))
 *   w_codes    [N][K/2]  u8    INT4 codes of R (two per byte, low nibble = even k)
 *   w_scales   [K/64][N] fp16  per (group, output channel): fp16(absmax/7)
 *   lora_down  [rank][K] bf16  L1^T (= U_r Sigma_r transposed); may be NULL if rank == 0
 *   lora_up    [N][rank] bf16  L2^T (= V_r); may be NULL if rank == 0
 * with W_hat = diag(1/fp64(smooth_inv)) W, L1 L2 = top-r SVD of W_hat
 * (randomized block subspace iteration with a one-sided Jacobi SVD of the
 * projected block, fp64), R = W_hat - bf16(L1) bf16(L2) in fp64, and codes
 * q = clamp(rne(R / s), -8, 7).  Returns SVDQ_ERR_NUMERIC on non-finite input,
 * an fp16 scale overflow or a non-converged SVD. */
int svdq_prepare_weights(const uint16_t* weight, int K, int N,
                         const float* act_absmax, float alpha, int rank, int group,
                         float* smooth_inv, uint8_t* w_codes, uint16_t* w_scales,
                         uint16_t* lora_down, uint16_t* lora_up);

/* As svdq_prepare_weights, with three extras:
 *   lora_down_in [rank][K], lora_up_in [N][rank] (bf16, both or neither):
 *       when given, the SVD is skipped and these factors are used (and copied
 *       to lora_down / lora_up); the residual is taken against them.
 *   sigma_out [rank] fp64 (nullable): the singular values of the split.
 *   power_iters (<= 0: default 8) subspace iterations; seed: RNG seed of the
 *       starting block (counter-based splitmix64 + Box-Muller). */
int svdq_prepare_weights_ex(const uint16_t* weight, int K, int N,
                            const float* act_absmax, float alpha, int rank, int group,
                            const uint16_t* lora_down_in, const uint16_t* lora_up_in,
                            int power_iters, uint64_t seed,
                            float* smooth_inv, uint8_t* w_codes, uint16_t* w_scales,
                            uint16_t* lora_down, uint16_t* lora_up, double* sigma_out);

/* Device, asynchronous.  Kernel 1: fused smoothing + per-(token, group of 64)
 * symmetric INT4 activation quantizer + low-rank down projection, reading
 * each input element from HBM once (model card, "Nunchaku Engine Design":
 * the down projection and the quantizer share their input).
 *
 *   x          [M][K]      bf16  input activations (with act = GELU_TANH,
 *                                tanh-GELU is applied to x first, in fp32,
 *                                as x / (1 + 2^(x (c1 + c3 x^2))) with the
 *                                hardware exp2 and reciprocal: the same
 *                                function, ~1e-6 relative, so a code may
 *                                differ by one from an fp64 GELU's where a
 *                                value sits on a rounding boundary)
 *   smooth_inv [K]         fp32
 *   lora_down  [rank][K]   bf16  (NULL allowed when rank == 0)
 * Outputs:
 *   x_codes    [M][K/2]    u8    codes q = clamp(rne(fp32(x_hat * fp32(1/s))), -8, 7)
 *   x_scales   [K/64][M]   fp16  s = fp16(fp32(absmax(x_hat over the group) / 7));
 *                                an all-zero group gets s = 0 and codes 0
 *   lora_act   [M][rank]   fp32  sum_k bf16(x_hat[m,k]) * lora_down[j][k]
 *                                (NULL allowed when rank == 0)
 * with x_hat = fp32(act(x) * smooth_inv).  |x_hat| above 7 * 65504 in a
 * group overflows the fp16 scale to inf (codes 0); such inputs are outside
 * the supported range.  K is limited to 32768 (smooth_inv is staged in LDS);
 * larger K returns SVDQ_ERR_UNSUPPORTED_SHAPE. */
int svdq_quant_act_lora_down(const void* x, const float* smooth_inv, const void* lora_down,
                             int M, int K, int rank, int group, int act,
                             void* x_codes, void* x_scales, float* lora_act,
                             void* stream);

/* Device, asynchronous.  Kernel 2: W4A4 GEMM on int8 MFMA with exact int32
 * per-group products, per-group dequantization, and the up projection plus
 * bias in the same fp32 accumulators (model card, "Nunchaku Engine Design":
 * the up projection and the 4-bit compute share their output).
 *
 *   x_codes  [M][K/2] u8, x_scales [K/64][M] fp16  (from kernel 1)
 *   w_codes  [N][K/2] u8, w_scales [K/64][N] fp16  (from preparation)
 *   lora_act [M][rank] fp32, lora_up [N][rank] bf16 (NULL allowed when rank == 0)
 *   bias     [N] bf16 or NULL
 * Output:
 *   y        [M][N] bf16 (out_dtype = SVDQ_OUT_BF16) or fp32 (SVDQ_OUT_F32):
 *            y = sum_g s_x[m,g] s_w[g,n] P_g[m,n]
 *                + sum_j bf16(lora_act[m,j]) lora_up[n][j] + bias[n],
 *            P_g = sum over the 64 k of group g of q_x q_w (exact int32),
 *            accumulated in fp32 over g in increasing order, rounded to the
 *            output type to nearest even.  Where the bias and the up
 *            projection enter that fp32 sum depends on the tile form the
 *            launch picks (first for 256 x 256 tiles, used when M is even and
 *            there are at least 192 of them; last for 128 x 128 tiles); both
 *            orders are within the rounding of the fp32 sum. */
int svdq_gemm_w4a4_lora_up(const void* x_codes, const void* x_scales,
                           const void* w_codes, const void* w_scales,
                           const float* lora_act, const void* lora_up, const void* bias,
                           int M, int N, int K, int rank, int group, int out_dtype,
                           void* y, void* stream);

/* Device, asynchronous.  Kernel 2 with the fused QKV epilogue: the operator
 * that consumes the QKV projection, the Q/K normalization and the rotary
 * embedding together ("Bringing Nunchaku 4-bit Diffusion Inference to
 * Diffusers", "Quantizing models with structural rewrites").  The weight is
 * the concatenation [W_q; W_k; W_v] along the output dimension (in that
 * order), so N = 3 * heads * 128 (head dimension SVDQ_QKV_HEAD_DIM).  After
 * the projection (exactly as svdq_gemm_w4a4_lora_up, bias included, in
 * fp32), every Q head and every K head h of row m is
 *     t = y[m, head] / sqrt(mean(y[m, head]^2) + eps) * g      (g = norm_q or norm_k)
 * then, when rope_cos / rope_sin are given, each adjacent pair (2i, 2i+1)
 * of the head turns by the row's angle i:
 *     (t0, t1) -> (t0 cos - t1 sin, t1 cos + t0 sin),  cos = rope_cos[m][i], sin = rope_sin[m][i].
 * V heads are stored as projected.  One rounding to the output type at the end.
 *   norm_q, norm_k [128] bf16    RMSNorm weights
 *   rope_cos, rope_sin [M][64] fp32 (both NULL: no rotation)
 *   eps >= 0 (finite)
 * Other arguments, layouts and errors as svdq_gemm_w4a4_lora_up; N not a
 * multiple of 384, or rotary tables of 2 GiB or more (M * 256 bytes), return
 * SVDQ_ERR_UNSUPPORTED_SHAPE. */
int svdq_gemm_w4a4_lora_up_qkv(const void* x_codes, const void* x_scales,
                               const void* w_codes, const void* w_scales,
                               const float* lora_act, const void* lora_up, const void* bias,
                               const void* norm_q, const void* norm_k,
                               const float* rope_cos, const float* rope_sin, float eps,
                               int M, int N, int K, int rank, int group, int out_dtype,
                               void* y, void* stream);

/* Device, asynchronous.  The unfused low-rank branch, kept as the reference
 * for the fusion the model card's "Nunchaku Engine Design" describes (its
 * section (a): running the rank-32 branch naively costs an extra read of
 * the 16-bit input for the down projection and an extra write of the 16-bit
 * output for the up projection).  Used with the two kernels above at
 * rank 0, they compute the same layer with those extra HBM passes:
 *
 * svdq_lora_down: lora_act [M][rank] fp32 = sum_k bf16(x_hat[m,k]) *
 *   lora_down[j][k], x_hat = fp32(act(x) * smooth_inv), reading x [M][K]
 *   bf16 again (no codes or scales are written).  Same limits as
 *   svdq_quant_act_lora_down; rank >= 16.
 * svdq_lora_up_add: y [M][N] bf16, read and rewritten in place:
 *   y = bf16(y + sum_j bf16(lora_act[m,j]) * lora_up[n][j]).  rank >= 16. */
int svdq_lora_down(const void* x, const float* smooth_inv, const void* lora_down, int M, int K,
                   int rank, int group, int act, float* lora_act, void* stream);
int svdq_lora_up_add(const float* lora_act, const void* lora_up, int M, int N, int rank, void* y,
                     void* stream);

/* ------------------------------------------------------------------------
 * The INT4 layer on the 6-bit matrix cores.  gfx950 has no INT4 MFMA; its
 * int8 MFMA is the 5.0 POPS path, its 6-bit float MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4) the 10 PFLOPS path.  Every INT4 code
 * q in [-8, 7] is exactly a value of the 6-bit float format E3M2 (sign,
 * 3 exponent bits with bias 3, 2 mantissa bits), and the MFMA's 64 exact
 * products of one group sum exactly in its fp32 accumulator, so the
 * per-group integer product P_g of the W4A4 GEMM (model card, "Nunchaku
 * Engine Design": 4-bit compute fused with the up projection) comes out bit
 * for bit as the integer result.  The entry points below compute the same
 * layer as svdq_quant_act_lora_down + svdq_gemm_w4a4_lora_up -- the same
 * codes, scales, products and dequantization -- with the codes carried in
 * 6-bit fields (0.75 byte per code instead of 0.5) laid out as the MFMA
 * reads them.
 *
 * Fragment layout of a [rows][K] code matrix: [K/64][RB][1536 bytes], one
 * 1536-byte fragment per (group g of 64 k, row block rb of 32 rows).  Lane
 * l = r + 32 h (r = 0..31, h = 0..1) of a fragment holds the 32 codes
 * k = 64 g + 32 h + j (j = 0..31) of the row in slot r, as a 192-bit
 * little-endian string with code j in bits 6j .. 6j + 5; the string's
 * dwords 0..3 are stored at byte 16 l of the fragment and dwords 4..5 at
 * byte 1024 + 8 l.  Code values: E3M2 bit patterns (0 = +0 for q = 0).
 *   SVDQ_FP6_ACTIVATIONS: slot r of row block rb is row 32 rb + r;
 *       RB = ceil(rows / 32).
 *   SVDQ_FP6_WEIGHTS: rows are grouped in panels of 128; slot r of row
 *       block 4 p + t is row 128 p + 4 r + t; RB = 4 ceil(rows / 128).
 * Slots past the last row hold +0.
 * ------------------------------------------------------------------------ */
enum { SVDQ_FP6_ACTIVATIONS = 0, SVDQ_FP6_WEIGHTS = 1 };

/* Bytes of a fragment-layout buffer: (K/64) * RB * 1536.  K % 64 != 0 returns
 * SVDQ_ERR_UNSUPPORTED_SHAPE; rows < 0, K <= 0, an unknown layout or a NULL
 * bytes_out SVDQ_ERR_INVALID_ARG. */
int svdq_fp6_operand_bytes(int rows, int K, int layout, size_t* bytes_out);

/* Host, synchronous.  Re-packs nibble codes (codes [rows][K/2] u8, two's
 * complement, low nibble = even k, as svdq_prepare_weights writes w_codes)
 * into the fragment layout `layout` (out: caller-owned host buffer of
 * svdq_fp6_operand_bytes bytes).  Used once per layer for the weights
 * (layout SVDQ_FP6_WEIGHTS). */
int svdq_pack_fp6_operand(const uint8_t* codes, int rows, int K, int layout, uint8_t* out);

/* Device, asynchronous.  Kernel 1 writing the codes in the fragment layout:
 * the same smoothing, quantizer, scales and down projection as
 * svdq_quant_act_lora_down (the same kernel, another store of the codes).
 *   x [M][K] bf16, smooth_inv [K] fp32, lora_down [rank][K] bf16 (NULL if
 *   rank == 0), act SVDQ_ACT_NONE or SVDQ_ACT_GELU_TANH.
 * Outputs:
 *   x_fp6    fragment layout SVDQ_FP6_ACTIVATIONS, (K/64) * ceil(M/32) * 1536
 *            bytes; rows M .. 32 ceil(M/32) - 1 are written as +0 codes
 *   x_scales [K/64][Mp] fp16 with Mp = 32 ceil(M/32) (padded rows: 0)
 *   lora_act [M][rank] fp32 (NULL if rank == 0)
 * Errors as svdq_quant_act_lora_down; buffers of 2 GiB or more return
 * SVDQ_ERR_UNSUPPORTED_SHAPE. */
int svdq_quant_act_lora_down_fp6(const void* x, const float* smooth_inv, const void* lora_down,
                                 int M, int K, int rank, int group, int act,
                                 void* x_fp6, void* x_scales, float* lora_act, void* stream);

/* Device, asynchronous.  Kernel 2 on the 6-bit MFMA: the output of
 * svdq_gemm_w4a4_lora_up for the same codes and scales,
 *   y = sum_g s_x[m,g] s_w[g,n] P_g[m,n] + sum_j bf16(lora_act[m,j]) lora_up[n][j] + bias[n],
 * accumulated in fp32: the groups in increasing g, each as
 * fma(P_g * s_x, s_w, acc) (P_g * s_x is exact), then the up projection 16
 * ranks at a time, then the bias; rounded to bf16 to nearest even (or
 * stored fp32).
 *   x_fp6    SVDQ_FP6_ACTIVATIONS layout of the activation codes,
 *   x_scales [K/64][Mp] fp16, Mp = 32 ceil(M/32)   (both from kernel 1)
 *   w_fp6    SVDQ_FP6_WEIGHTS layout of the weight codes (svdq_pack_fp6_operand),
 *   w_scales [K/64][N] fp16, lora_act [M][rank] fp32, lora_up [N][rank]
 *   bf16 (NULL if rank == 0), bias [N] bf16 or NULL.
 * Shape rules and errors as svdq_gemm_w4a4_lora_up; every buffer, y
 * included, must be under 2 GiB (the kernel addresses them with 32-bit
 * offsets), else SVDQ_ERR_UNSUPPORTED_SHAPE. */
int svdq_gemm_w4a4_fp6_lora_up(const void* x_fp6, const void* x_scales,
                               const void* w_fp6, const void* w_scales,
                               const float* lora_act, const void* lora_up, const void* bias,
                               int M, int N, int K, int rank, int group, int out_dtype,
                               void* y, void* stream);

/* Device, asynchronous.  The same layer as svdq_gemm_w4a4_fp6_lora_up (the
 * same sum, each group as fma(P_g * s_w, s_x, acc), then the up projection
 * 16 ranks at a time, then the bias; one rounding), computed in 256 x 192
 * output tiles: for layers whose 256 x 256 tiles would leave CUs idle (N =
 * 3072 at M = 4096: 192 tiles of 256 x 256, 256 of 256 x 192).
 *   w_fp6    the weight codes in the SVDQ_FP6_ACTIVATIONS layout (plain row
 *            blocks of 32 channels; svdq_pack_fp6_operand with that layout),
 *   other arguments and layouts as svdq_gemm_w4a4_fp6_lora_up.
 * N must be a multiple of 192, else SVDQ_ERR_UNSUPPORTED_SHAPE; other errors
 * as svdq_gemm_w4a4_fp6_lora_up. */
int svdq_gemm_w4a4_fp6_lora_up_n192(const void* x_fp6, const void* x_scales,
                                    const void* w_fp6, const void* w_scales,
                                    const float* lora_act, const void* lora_up, const void* bias,
                                    int M, int N, int K, int rank, int group, int out_dtype,
                                    void* y, void* stream);

/* Host.  1 when svdq_gemm_w4a4_fp6_lora_up_n192 is expected to be faster
 * than svdq_gemm_w4a4_fp6_lora_up for an M x N output on the current device
 * (N % 192 == 0 and less time in rounds of tiles over the CUs, counting a
 * 256 x 192 tile as 0.875 of a 256 x 256 one), else 0. */
int svdq_fp6_n192_preferred(int M, int N);

/* Host.  The kernels expected to be fastest for an INT4 layer's M x N output
 * on the current device: 0 = svdq_quant_act_lora_down_fp6 +
 * svdq_gemm_w4a4_fp6_lora_up (256 x 256 tiles), 1 = the same kernel 1 +
 * svdq_gemm_w4a4_fp6_lora_up_n192, 2 = the int8 engine
 * (svdq_quant_act_lora_down + svdq_gemm_w4a4_lora_up, whose 128 x 128 form
 * keeps more CUs busy when 256 x 256 tiles would cover fewer than half of
 * them).  All three compute the same layer. */
int svdq_int4_route(int M, int N);

/* Device, asynchronous.  The fused QKV operator of svdq_gemm_w4a4_lora_up_qkv
 * (the same per-head RMSNorm of the Q and K heads and rotary embedding of
 * their adjacent pairs, the same argument meanings) on the 6-bit MFMA: the
 * projection is that of svdq_gemm_w4a4_fp6_lora_up in every bit, bias
 * included, so the V columns equal its output exactly; the Q and K heads
 * are then normalized and rotated in fp32 before the one rounding.
 *   x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias as
 *   svdq_gemm_w4a4_fp6_lora_up; norm_q, norm_k, rope_cos, rope_sin, eps as
 *   svdq_gemm_w4a4_lora_up_qkv.
 * Errors: those of both; rotary tables of 2 GiB or more (M * 256 bytes)
 * return SVDQ_ERR_UNSUPPORTED_SHAPE. */
int svdq_gemm_w4a4_fp6_lora_up_qkv(const void* x_fp6, const void* x_scales,
                                   const void* w_fp6, const void* w_scales,
                                   const float* lora_act, const void* lora_up, const void* bias,
                                   const void* norm_q, const void* norm_k,
                                   const float* rope_cos, const float* rope_sin, float eps,
                                   int M, int N, int K, int rank, int group, int out_dtype,
                                   void* y, void* stream);

/* ------------------------------------------------------------------------
 * The MLP chain (SVDQuant pages: "Introducing Nunchaku Lite", the fused
 * GELU/MLP kernels of the original engine).  An MLP pair is an up layer
 * (K -> N) whose output, through tanh-GELU, is the input of a down layer
 * (N -> N2).  The chain runs the up layer's kernel 2 on the 6-bit MFMA and,
 * in its epilogue, the down layer's kernel 1 on the tile it just computed:
 * Y_up never goes to memory.  For every row m and group g of 64 of the up
 * layer's N columns:
 *   x = bf16(Y_up[m, n])  (Y_up as svdq_gemm_w4a4_fp6_lora_up computes it),
 *   x_hat = fp32(gelu_tanh(x) * smooth_inv_dn[n]), then the INT4 quantizer
 *   of svdq_quant_act_lora_down_fp6: codes into x_fp6_dn, scales into
 *   x_scales_dn -- bit for bit what the two-layer path writes;
 * and lora_act_dn = sum over the column slices c of 256 columns, in slice
 * order in fp32, of fp32( bf16(x_hat[:, c]) lora_down_dn[:, c]^T ) -- the
 * whole-row down projection up to the fp32 rounding of each slice's partial.
 * The down layer then runs svdq_gemm_w4a4_fp6_lora_up on these outputs.
 * ------------------------------------------------------------------------ */

/* Host.  Workspace bytes of svdq_gemm_w4a4_fp6_mlp_chain: the partial down
 * projections, ceil(N/256) * M * rank_dn fp32 (0 when rank_dn == 0).
 * SVDQ_ERR_INVALID_ARG for negative sizes or a NULL bytes_out. */
int svdq_mlp_chain_workspace_bytes(int M, int N, int rank_dn, size_t* bytes_out);

/* Device, asynchronous; two kernels on `stream`.  Up layer (shapes and
 * layouts as svdq_gemm_w4a4_fp6_lora_up): x_fp6, x_scales, w_fp6,
 * w_scales, lora_act, lora_up, bias, M, N, K, rank, group.  Down layer:
 *   smooth_inv_dn  [N] fp32          its 1 / lambda
 *   lora_down_dn   [rank_dn][N] bf16 its L1^T (NULL if rank_dn == 0)
 * Outputs (caller-owned device memory, the down layer's kernel-1 outputs):
 *   x_fp6_dn    SVDQ_FP6_ACTIVATIONS layout, [N/64][ceil(M/32)][1536] u8
 *   x_scales_dn [N/64][Mp] fp16, Mp = 32 ceil(M/32) (rows M..Mp-1 zero)
 *   lora_act_dn [M][rank_dn] fp32 (NULL if rank_dn == 0)
 *   workspace   svdq_mlp_chain_workspace_bytes() bytes, 16-byte aligned
 *               (NULL if rank_dn == 0); its contents afterwards are
 *               unspecified.  Calls that share a workspace must not overlap.
 * Requires N % 64 == 0 (the down layer's K), rank_dn % 16 == 0,
 * 0 <= rank_dn <= min(N, SVDQ_MAX_RANK); other shape rules and errors as
 * svdq_gemm_w4a4_fp6_lora_up; SVDQ_ERR_INVALID_ARG for a workspace smaller
 * than required. */
int svdq_gemm_w4a4_fp6_mlp_chain(const void* x_fp6, const void* x_scales,
                                 const void* w_fp6, const void* w_scales,
                                 const float* lora_act, const void* lora_up, const void* bias,
                                 int M, int N, int K, int rank, int group,
                                 const float* smooth_inv_dn, const void* lora_down_dn, int rank_dn,
                                 void* x_fp6_dn, void* x_scales_dn, float* lora_act_dn,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Device, asynchronous.  svdq_gemm_w4a4_fp6_mlp_chain without the workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * partial down projections go to a device-resident scratch array of
 * SVDQ_CHAIN_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends (its address is looked up once per device, on
 * the first call there).  The call allocates nothing.  Returns
 * SVDQ_ERR_UNSUPPORTED_SHAPE when svdq_mlp_chain_workspace_bytes() exceeds
 * SVDQ_CHAIN_SCRATCH_BYTES; every other rule and error as
 * svdq_gemm_w4a4_fp6_mlp_chain.  All calls on one device share that
 * device's scratch, which keeps the last call's contents: calls that
 * overlap on one device (on different streams, or otherwise unordered)
 * race.  Nothing in it needs to start at zero: each call writes every
 * partial it reads. */
#define SVDQ_CHAIN_SCRATCH_BYTES (32u << 20)
int svdq_gemm_w4a4_fp6_mlp_chain_noalloc(const void* x_fp6, const void* x_scales,
                                         const void* w_fp6, const void* w_scales,
                                         const float* lora_act, const void* lora_up, const void* bias,
                                         int M, int N, int K, int rank, int group,
                                         const float* smooth_inv_dn, const void* lora_down_dn, int rank_dn,
                                         void* x_fp6_dn, void* x_scales_dn, float* lora_act_dn, void* stream);

/* ------------------------------------------------------------------------
 * 4-bit float variant (MXFP4).  The pages offer the layer with INT4 and with
 * 4-bit float operands ("Bringing Nunchaku 4-bit Diffusion Inference to
 * Diffusers", "Background: SVDQuant and Nunchaku"; the ``precision`` field
 * of "Native loading in Diffusers").  The float encoding here is the one
 * gfx950's matrix cores apply natively, OCP Microscaling MXFP4: FP4 E2M1
 * elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; two per byte, low nibble
 * = even k, sign in bit 3) with one E8M0 scale byte 2^(s - 127) per block of
 * 32 consecutive k.  A block's scale is 2^e, e = floor(log2(amax)) - 2
 * clamped to [-127, 127] (e = -127 for an all-zero block); elements are
 * v / 2^e rounded to nearest E2M1 with ties to the even code and saturation
 * at 6, and a value that rounds to zero is code 0.  Smoothing, the low-rank
 * branch and the conventions above are those of the INT4 layer.  K must be
 * a multiple of 128 (and at most 32768 for the activation kernel).
 * ------------------------------------------------------------------------ */

/* Bytes of one MXFP4-prepared layer: codes N*K/2 + scales (K/32)*N + bf16
 * factors 2*rank*(K+N) + fp32 smooth_inv 4*K. */
int svdq_prepared_bytes_mxfp4(int K, int N, int rank, size_t* bytes_out);

/* Host, synchronous.  As svdq_prepare_weights_ex with the residual R
 * quantized to MXFP4 per (output channel, block of 32 along K):
 *   w_codes  [N][K/2]  u8  E2M1 codes
 *   w_scales [N][K/32] u8  E8M0 scales, row-major per output channel */
int svdq_prepare_weights_mxfp4(const uint16_t* weight, int K, int N,
                               const float* act_absmax, float alpha, int rank,
                               const uint16_t* lora_down_in, const uint16_t* lora_up_in,
                               int power_iters, uint64_t seed,
                               float* smooth_inv, uint8_t* w_codes, uint8_t* w_scales,
                               uint16_t* lora_down, uint16_t* lora_up, double* sigma_out);

/* Device, asynchronous.  Kernel 1 with the MXFP4 quantizer: x_hat as for
 * INT4 (fp32), then per (token, block of 32) the block scale and E2M1 codes
 * above; the down projection is unchanged.
 *   x_codes  [M][K/2]  u8  E2M1 codes
 *   x_scales [M][K/32] u8  E8M0 scales, row-major per token
 *   lora_act [M][rank] fp32 (NULL allowed when rank == 0) */
int svdq_quant_act_lora_down_mxfp4(const void* x, const float* smooth_inv, const void* lora_down,
                                   int M, int K, int rank, int act,
                                   void* x_codes, void* x_scales, float* lora_act, void* stream);

/* Device, asynchronous.  Kernel 2 for MXFP4 operands on the block-scaled FP4
 * MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), which applies both scales and
 * accumulates in fp32:
 *   y = sum_b 2^(ex[m,b] + ew[n,b]) sum_{k in b} qx[m,k] qw[n,k]
 *       + sum_j bf16(lora_act[m,j]) lora_up[n][j] + bias[n],
 * rounded to bf16 (or stored fp32).  The MFMA's summation order inside an
 * instruction is the hardware's; across instructions k increases. */
int svdq_gemm_mxfp4_lora_up(const void* x_codes, const void* x_scales,
                            const void* w_codes, const void* w_scales,
                            const float* lora_act, const void* lora_up, const void* bias,
                            int M, int N, int K, int rank, int out_dtype,
                            void* y, void* stream);

/* ------------------------------------------------------------------------
 * AWQ W4A16 linear: 4-bit weights, 16-bit activations, for the adaptive
 * normalization / modulation projections ("Bringing Nunchaku 4-bit Diffusion
 * Inference to Diffusers", "Introducing Nunchaku Lite"; int4, group 64 in
 * "Native loading in Diffusers").  These layers see a few rows (the
 * conditioning vectors), so the path streams the weight once at HBM rate.
 * ------------------------------------------------------------------------ */

/* Host, synchronous.  Activation-aware weight quantization of one layer.
 *   weight [N][K] bf16, x_cal [Mc][K] bf16 calibration activations
 *   alpha: < 0 searches {k / 20.0 : k = 0..19} (fp64); otherwise used as given (< 1)
 * Channel scale t_k = max(a_k, 1e-4)^alpha / sqrt(max t * min t) with
 * a_k = mean_m |x_cal[m][k]|; alpha minimizes the calibration output error
 * sum (x_cal W^T - x_cal diag(t)^-1 Q(W diag(t))^T)^2 (first minimum).
 * Per (output channel, group of 64) of W diag(t), t := 1 / fp64(inv_scale):
 * s = fp16(max(max - min, 1e-5) / 15), z = clamp(rne(-min / s), 0, 15),
 * q = clamp(rne(w / s) + z, 0, 15).  Outputs (caller-owned host buffers):
 *   inv_scale [K] fp32 (1 / t), w_codes [N][K/2] u8 (unsigned codes, low
 *   nibble = even k), w_scales [N][K/64] fp16, w_zeros [N][K/64] u8,
 *   alpha_out (nullable).  N % 32 == 0, K % 64 == 0. */
int svdq_awq_prepare(const uint16_t* weight, int K, int N, const uint16_t* x_cal, int Mc, double alpha,
                     int group, float* inv_scale, uint8_t* w_codes, uint16_t* w_scales,
                     uint8_t* w_zeros, double* alpha_out);

/* Device, asynchronous.  x_hat [M][K] bf16 = bf16(fp32(x * inv_scale)) and
 * xsum [K/64][16] fp32: per group and row, the sum of the group's x_hat in
 * increasing k (rows M..15 are written as 0).  M <= 16. */
int svdq_awq_quant_act(const void* x, const float* inv_scale, int M, int K, void* x_hat, float* xsum,
                       void* stream);

/* Device, asynchronous.  y [M][N] bf16 = bf16(sum_g s[n][g] (sum_{k in g}
 * q[n][k] x_hat[m][k] - z[n][g] xsum[g][m]) + bias[n]) with fp32 sums; the
 * inner sums run on bf16 MFMA, or for one row with K <= 8192 on bf16 dot
 * products into fp32 (as sum (128 + q) x_hat - (128 + z) xsum in both).
 * M <= 16, N % 32 == 0, K % 64 == 0; bias nullable. */
int svdq_awq_gemv(const void* x_hat, const float* xsum, const void* w_codes, const void* w_scales,
                  const void* w_zeros, const void* bias, int M, int N, int K, void* y, void* stream);

/* Device, asynchronous.  One row (the modulation layers' single
 * conditioning vector): y [N] bf16 = what svdq_awq_quant_act followed by
 * svdq_awq_gemv produce for M = 1 from x [K] bf16 and inv_scale [K] fp32,
 * bit for bit, in one launch (x_hat and the group sums are formed on the
 * device per block, in the same arithmetic and order).  K <= SVDQ_AWQ_ROW_MAX_K,
 * K % 64 == 0, N % 32 == 0; bias nullable; buffers 16-byte aligned. */
int svdq_awq_linear_row(const void* x, const float* inv_scale, const void* w_codes, const void* w_scales,
                        const void* w_zeros, const void* bias, int N, int K, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
