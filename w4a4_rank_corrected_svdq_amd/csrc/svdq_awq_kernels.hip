// HIP kernels for the AWQ W4A16 linear on gfx950: 4-bit weights, 16-bit
// activations, few rows ("Bringing Nunchaku 4-bit Diffusion Inference to
// Diffusers", "Introducing Nunchaku Lite": the modulation projections,
// memory-bound and precision-sensitive; "Native loading in Diffusers": int4,
// group 64).  The weight read dominates, so the path is built to stream it
// from HBM at full rate.
//
// k_awq_act: x_hat = bf16(fp32(x * inv_scale)) [M][K] and, per (group of 64,
//   row), X_g = sum of the group's x_hat values in fp32 in increasing k,
//   laid out [K/64][16] (rows M..15 zero).
// k_awq_gemv: Y = bf16(sum_g s_g (sum_{k in g} q x_hat - z_g X_g) + bias) for
//   M <= 16 rows.  The inner sums run on bf16 MFMA 16x16x32: a nibble q
//   becomes the bf16 value 128 + q by OR-ing it into the bit pattern 0x4300
//   (128 = 1.0 x 2^7 has seven free mantissa bits), so one MFMA pair per group
//   gives D = sum (128 + q) x_hat exactly per product, and the kernel
//   subtracts (128 + z_g) X_g.  A wave owns 16 output columns and a quarter of
//   K; the four waves of a block split K and add their partial results in LDS
//   in wave order.  Every weight load of a wave's K range is issued before
//   any is used, which keeps enough bytes in flight to stream HBM.
//
// MFMA 16x16x32 bf16 layouts (wave64): A lane l holds row l % 16, 8 values
// of k chosen by l / 16; B lane l holds column l % 16 and the same k; D lane
// l holds column l % 16, rows 4 (l / 16) + i.  Here rows are the M input
// rows, columns the output channels, and lane group h = l / 16 takes k =
// 64 g + 16 h + 8 t + (0..7) in the t-th MFMA of group g (any permutation of
// k applied to both operands leaves the product unchanged), so each lane
// reads 8 contiguous code bytes per group.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq.h"
#include "svdq_device.h"
#include "svdq_internal.h"

namespace {

constexpr int AWQ_GROUP = 64;
constexpr int AWQ_COLS = 16;        // output columns per block
constexpr int AWQ_WAVES = 4;        // K split per block
constexpr int AWQ_CHUNK = 16;       // groups whose weight loads are in flight together
constexpr int AWQ_MAX_ROWS = 16;

__global__ __launch_bounds__(256) void k_awq_act(const uint16_t* __restrict__ x, const float* __restrict__ inv_scale,
                                                 int M, int K, uint16_t* __restrict__ x_hat,
                                                 float* __restrict__ xsum) {
  const int G = K / AWQ_GROUP;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;      // (group, row) pair, row-fastest
  if (t >= G * AWQ_MAX_ROWS) return;
  const int g = t / AWQ_MAX_ROWS, m = t % AWQ_MAX_ROWS;
  float s = 0.f;
  if (m < M) {
    const uint16_t* xr = x + static_cast<size_t>(m) * K + g * AWQ_GROUP;
    uint16_t* hr = x_hat + static_cast<size_t>(m) * K + g * AWQ_GROUP;
    for (int i = 0; i < AWQ_GROUP; ++i) {
      const uint32_t b = f32_to_bf16_bits(bf16_bits_to_f32(xr[i]) * inv_scale[g * AWQ_GROUP + i]);
      hr[i] = static_cast<uint16_t>(b);
      s += bf16_bits_to_f32(b);
    }
  }
  xsum[t] = s;
}

// 8 nibbles (low nibble first) -> 8 bf16 values 128 + q, as four dwords.
__device__ __forceinline__ v8bf awq_nibbles_to_bf16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d[i] = __builtin_amdgcn_perm(hi, lo, static_cast<uint32_t>(i | (0x0C << 8) | ((4 + i) << 16) | (0x0C << 24))) |
           0x43004300u;
  return __builtin_bit_cast(v8bf, make_uint4(d[0], d[1], d[2], d[3]));
}

__global__ __launch_bounds__(AWQ_WAVES * 64) void k_awq_gemv(
    const uint16_t* __restrict__ x_hat, const float* __restrict__ xsum, const uint8_t* __restrict__ w_codes,
    const _Float16* __restrict__ w_scales, const uint8_t* __restrict__ w_zeros, const uint16_t* __restrict__ bias,
    int M, int N, int K, uint16_t* __restrict__ y) {
  __shared__ float part[AWQ_WAVES][64][4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, h = lane >> 4;
  const int n = blockIdx.x * AWQ_COLS + col;                 // N % 16 == 0: always < N
  const int G = K / AWQ_GROUP;
  const int per = (G + AWQ_WAVES - 1) / AWQ_WAVES;
  const int g_begin = wave * per, g_end = min(G, g_begin + per);
  const uint32_t Kb = static_cast<uint32_t>(K) / 2;

  const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(w_codes), 0, static_cast<int>(static_cast<size_t>(N) * Kb), 0x00020000);
  // activation rows past M read as zero
  const __amdgpu_buffer_rsrc_t x_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x_hat), 0, static_cast<int>(static_cast<size_t>(M) * K * 2), 0x00020000);
  const uint32_t w_row = static_cast<uint32_t>(n) * Kb + 8u * h;
  const uint32_t x_row = static_cast<uint32_t>(col) * K * 2 + 32u * h;   // A operand row = lane % 16

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = g_begin; c0 < g_end; c0 += AWQ_CHUNK) {
    uint2 wv[AWQ_CHUNK];
#pragma unroll
    for (int c = 0; c < AWQ_CHUNK; ++c) {
      const int g = c0 + c;
      wv[c] = make_uint2(0, 0);
      if (g < g_end)
        wv[c] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(w_rs, w_row + 32u * g, 0, 0));
    }
#pragma unroll
    for (int c = 0; c < AWQ_CHUNK; ++c) {
      const int g = c0 + c;
      if (g >= g_end) break;
      const uint32_t xo = x_row + 128u * g;
      const v8bf a0 = __builtin_bit_cast(v8bf, __builtin_amdgcn_raw_buffer_load_b128(x_rs, xo, 0, 0));
      const v8bf a1 = __builtin_bit_cast(v8bf, __builtin_amdgcn_raw_buffer_load_b128(x_rs, xo + 16u, 0, 0));
      v4f d = {0.f, 0.f, 0.f, 0.f};
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, awq_nibbles_to_bf16(wv[c].x), d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, awq_nibbles_to_bf16(wv[c].y), d, 0, 0, 0);
      const float s = static_cast<float>(w_scales[static_cast<size_t>(n) * G + g]);
      const float cz = 128.0f + static_cast<float>(w_zeros[static_cast<size_t>(n) * G + g]);
      const float4 xs = *reinterpret_cast<const float4*>(xsum + g * AWQ_MAX_ROWS + 4 * h);
      acc[0] = fmaf(s, fmaf(-cz, xs.x, d[0]), acc[0]);
      acc[1] = fmaf(s, fmaf(-cz, xs.y, d[1]), acc[1]);
      acc[2] = fmaf(s, fmaf(-cz, xs.z, d[2]), acc[2]);
      acc[3] = fmaf(s, fmaf(-cz, xs.w, d[3]), acc[3]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][lane][i] = acc[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = part[0][lane][i];
#pragma unroll
      for (int w = 1; w < AWQ_WAVES; ++w) v += part[w][lane][i];
      const int m = 4 * h + i;
      if (bias) v += bf16_bits_to_f32(bias[n]);
      if (m < M) y[static_cast<size_t>(m) * N + n] = static_cast<uint16_t>(f32_to_bf16_bits(v));
    }
  }
}

}  // namespace

namespace svdq {

int launch_awq_quant_act(const void* x, const float* inv_scale, int M, int K, void* x_hat, float* xsum,
                         void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int t = (K / AWQ_GROUP) * AWQ_MAX_ROWS;
  hipLaunchKernelGGL(k_awq_act, dim3((t + 255) / 256), dim3(256), 0, st, static_cast<const uint16_t*>(x), inv_scale,
                     M, K, static_cast<uint16_t*>(x_hat), xsum);
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

int launch_awq_gemv(const void* x_hat, const float* xsum, const void* w_codes, const void* w_scales,
                    const void* w_zeros, const void* bias, int M, int N, int K, void* y, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_awq_gemv, dim3(N / AWQ_COLS), dim3(AWQ_WAVES * 64), 0, st, static_cast<const uint16_t*>(x_hat),
                     xsum, static_cast<const uint8_t*>(w_codes), static_cast<const _Float16*>(w_scales),
                     static_cast<const uint8_t*>(w_zeros), static_cast<const uint16_t*>(bias), M, N, K,
                     static_cast<uint16_t*>(y));
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

}  // namespace svdq
