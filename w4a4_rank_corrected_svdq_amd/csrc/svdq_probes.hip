// Peak-rate probes for the measurement harness (not part of the layer): the
// dense matrix-core rates that the layer's kernels are priced against,
// measured on the device at hand next to the published figures.
//
// Each wave runs accumulation chains of one MFMA form for `iters`
// iterations on register operands (no memory traffic in the loop) and
// writes its accumulators to a sink buffer, so nothing is optimized away.
// The forms and chain counts are the fastest measured on gfx950 with every
// SIMD holding several waves: int8 peaks with the 32x32x32 form and one
// chain per wave (the 16x16x64 form stays near three quarters of that), FP4
// with the 32x32x64 form and four chains.  Three more kinds time the 6-bit
// route's inner loop: its FP6 MFMAs, its fp32 dequantization, and both
// interleaved as kernel 2 issues them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq.h"
#include "svdq_internal.h"
#include "svdq_probe.h"

#include "svdq_device.h"

namespace {

constexpr int PROBE_THREADS = 256;
constexpr int I8_CHAINS = 1;     // 32x32x32 int8: 16-register results
constexpr int FP4_CHAINS = 4;    // 32x32x64 FP4: 16-register results

__global__ __launch_bounds__(PROBE_THREADS) void k_probe_mfma_i8(int iters, v16i* __restrict__ sink) {
  const int t = threadIdx.x;
  const v4i a = v4i{t + 1, 3 * t + 5, 7, t ^ 0x55};
  const v4i b = v4i{2 * t + 3, 11, t ^ 0x33, t + 9};
  v16i d[I8_CHAINS];
#pragma unroll
  for (int c = 0; c < I8_CHAINS; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) d[c][e] = c + e;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < I8_CHAINS; ++c) d[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, d[c], 0, 0, 0);
  }
  v16i s = d[0];
#pragma unroll
  for (int c = 1; c < I8_CHAINS; ++c) s += d[c];
  sink[static_cast<size_t>(blockIdx.x) * PROBE_THREADS + t] = s;
}

__global__ __launch_bounds__(PROBE_THREADS) void k_probe_mfma_fp4(int iters, v16f* __restrict__ sink) {
  const int t = threadIdx.x;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (t * 0x01010101) ^ (i * 0x12345);
    b[i] = (t * 0x00FF00FF) ^ (i * 0x6789);
  }
  v16f d[FP4_CHAINS];
#pragma unroll
  for (int c = 0; c < FP4_CHAINS; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) d[c][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < FP4_CHAINS; ++c)
      // cbsz = blgp = 4: both operands FP4 E2M1; E8M0 scales 127 (= 1)
      d[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, d[c], 4, 4, 0, 127, 0, 127);
  }
  v16f s = d[0];
#pragma unroll
  for (int c = 1; c < FP4_CHAINS; ++c) s += d[c];
  sink[static_cast<size_t>(blockIdx.x) * PROBE_THREADS + t] = s;
}

// The 6-bit route's inner loop on registers: eight 32 x 32 tiles per
// iteration.  MODE 0: the FP6 MFMAs only (eight independent results); MODE 1:
// the dequantization only, on stand-in results; MODE 2: both, the MFMA of
// tile u issued before tile u - 1 is dequantized (the kernel's order).  The
// empty asm statements keep the compiler from merging the repeated MFMAs or
// hoisting loop-invariant work.
constexpr int MIX_TILES = 8;

template <int MODE>
__global__ __launch_bounds__(PROBE_THREADS, 2) void k_probe_fp6_mix(int iters, v16f* __restrict__ sink) {
  const int t = threadIdx.x;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = ((t * 0x01010101) ^ (i * 0x12345)) & 0x3DF7DF7D;
    b[i] = ((t * 0x00FF00FF) ^ (i * 0x6789)) & 0x3DF7DF7D;
  }
  float sx[16], sw[4];
#pragma unroll
  for (int i = 0; i < 16; ++i) sx[i] = 1.0f + 0.001f * i + 1e-6f * t;
#pragma unroll
  for (int i = 0; i < 4; ++i) sw[i] = 0.5f + 0.01f * i;
  v16f acc[MIX_TILES];
  v16f ch[MIX_TILES];
#pragma unroll
  for (int c = 0; c < MIX_TILES; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[c][e] = 0.f;
      ch[c][e] = static_cast<float>(t + e + c);
    }
  const v16f zero = {};
  v16f prev = ch[0];
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < MIX_TILES; ++u) {
      asm volatile("" : "+v"(a));
      v16f d;
      if (MODE == 1) {
        asm volatile("" : "+v"(ch[u & 1]));
        d = ch[u & 1];
      } else {
        // cbsz = blgp = 3: both operands FP6 E3M2; E8M0 scales 127 (= 1)
        d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, MODE == 0 ? ch[u] : zero, 3, 3, 0, 127, 0, 127);
      }
      if (MODE == 0) {
        ch[u] = d;
        continue;
      }
      const int pu = (u + MIX_TILES - 1) % MIX_TILES;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[pu][e] = __builtin_fmaf(prev[e] * sx[e], sw[pu & 3], acc[pu][e]);
      prev = d;
    }
  }
  v16f s = prev;
#pragma unroll
  for (int c = 0; c < MIX_TILES; ++c) s += acc[c] + ch[c];
  sink[static_cast<size_t>(blockIdx.x) * PROBE_THREADS + t] = s;
}

}  // namespace

namespace svdq {

int launch_probe_mfma(int kind, int blocks, int iters, void* sink, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  v16f* fs = static_cast<v16f*>(sink);
  if (kind == SVDQ_PROBE_MFMA_I8)
    hipLaunchKernelGGL(k_probe_mfma_i8, dim3(blocks), dim3(PROBE_THREADS), 0, st, iters, static_cast<v16i*>(sink));
  else if (kind == SVDQ_PROBE_MFMA_FP4)
    hipLaunchKernelGGL(k_probe_mfma_fp4, dim3(blocks), dim3(PROBE_THREADS), 0, st, iters, fs);
  else if (kind == SVDQ_PROBE_MFMA_FP6)
    hipLaunchKernelGGL(k_probe_fp6_mix<0>, dim3(blocks), dim3(PROBE_THREADS), 0, st, iters, fs);
  else if (kind == SVDQ_PROBE_DEQUANT)
    hipLaunchKernelGGL(k_probe_fp6_mix<1>, dim3(blocks), dim3(PROBE_THREADS), 0, st, iters, fs);
  else
    hipLaunchKernelGGL(k_probe_fp6_mix<2>, dim3(blocks), dim3(PROBE_THREADS), 0, st, iters, fs);
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

double probe_mfma_ops(int kind, int blocks, int iters) {
  const double waves = static_cast<double>(blocks) * (PROBE_THREADS / 64);
  if (kind == SVDQ_PROBE_MFMA_I8) return waves * iters * I8_CHAINS * (2.0 * 32 * 32 * 32);
  if (kind == SVDQ_PROBE_MFMA_FP4) return waves * iters * FP4_CHAINS * (2.0 * 32 * 32 * 64);
  if (kind == SVDQ_PROBE_DEQUANT) return waves * iters * MIX_TILES * (3.0 * 32 * 32);
  return waves * iters * MIX_TILES * (2.0 * 32 * 32 * 64);
}

}  // namespace svdq
