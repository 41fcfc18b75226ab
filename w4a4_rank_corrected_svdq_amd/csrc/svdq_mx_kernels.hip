// HIP kernel for the 4-bit float (MXFP4) variant of the SVDQuant W4A4 linear
// on gfx950.
//
// The pages offer the layer with INT4 and with 4-bit float operands
// ("Bringing Nunchaku 4-bit Diffusion Inference to Diffusers", "Background:
// SVDQuant and Nunchaku").  gfx950's matrix cores take FP4 E2M1 operands with
// one E8M0 scale per 32 consecutive k of each row (OCP Microscaling, MXFP4)
// and apply the scales inside v_mfma_scale_f32_32x32x64_f8f6f4, so the whole
// product sum_b 2^(ex + ew) <qx, qw>_b accumulates in the MFMA's fp32
// accumulators: there is no per-group dequantization on the vector ALUs,
// and packed codes are MFMA operands as they sit in memory.
//
// k_gemm_mxfp4_lora_up: Y = MXFP4 product + bf16(lora_act) L2 + bias.
//   Block tile 128 (m) x 256 (n), 4 waves in 2 x 2, wave tile 64 x 128 =
//   2 x 4 MFMA tiles of 32 x 32, computed transposed (weight rows are the
//   MFMA A operand, activation rows the B operand) so a lane ends with one
//   output row and runs of four output columns.  The K loop runs in stages
//   of 128 k (two MFMA k-steps of 64), loaded from HBM one stage ahead into
//   registers and stored to a double-buffered LDS tile; each fragment is one
//   16-byte LDS read.
//
// Operand layout of the 32x32x64 FP4 MFMA (wave64): lane l supplies row
// l % 32 and the 32 k of block l / 32 (16 bytes, element j in nibble j, low
// nibble first) together with that (row, block)'s E8M0 scale in its scale
// register; C/D as for every 32x32 MFMA: lane l holds column l % 32, rows
// 8b + 4(l / 32) + i in register 4b + i.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq.h"
#include "svdq_device.h"
#include "svdq_internal.h"

namespace {

constexpr int MX_BM = 128;                   // block tile rows (m)
constexpr int MX_BN = 256;                   // block tile columns (n)
constexpr int MX_WM = 64;                    // wave tile rows
constexpr int MX_WN = 128;                   // wave tile columns
constexpr int MX_TI = MX_WM / 32;            // 32x32 tiles per wave along m
constexpr int MX_TJ = MX_WN / 32;            // along n
constexpr int MX_KS = 128;                   // k per stage
constexpr int MX_THREADS = 256;

// LDS: codes as four 16-byte chunks per row and stage (chunk c = k 32c ..
// 32c + 31 of the stage = one MFMA block), chunk c of row r at position
// c ^ (((r >> 1) ^ (r >> 3)) & 3) so that fragment reads and loader writes
// spread over all banks; scales as one dword per row and stage (the four
// E8M0 bytes of the stage's blocks).
struct MxSmem {
  uint4 a[2][MX_BM][4];
  uint4 b[2][MX_BN][4];
  uint32_t sa[2][MX_BM];
  uint32_t sb[2][MX_BN];
};
constexpr size_t MX_SMEM_MAIN = sizeof(MxSmem);
constexpr size_t MX_SMEM_EPI = static_cast<size_t>(4) * MX_WM * MX_WN * 2;   // bf16 output tiles
constexpr size_t MX_SMEM = MX_SMEM_MAIN > MX_SMEM_EPI ? MX_SMEM_MAIN : MX_SMEM_EPI;

__device__ __forceinline__ int mx_swz(int row, int chunk) { return chunk ^ (((row >> 1) ^ (row >> 3)) & 3); }

template <int OUT_F32, int HAS_RANK>
__global__ __launch_bounds__(MX_THREADS, 2) void k_gemm_mxfp4_lora_up(
    const uint8_t* __restrict__ x_codes, const uint8_t* __restrict__ x_scales,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
    const float* __restrict__ lora_act, const uint16_t* __restrict__ lora_up,
    const uint16_t* __restrict__ bias, int M, int N, int K, int rank, void* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char mx_smem_raw[];
  MxSmem& sm = *reinterpret_cast<MxSmem*>(mx_smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nM = (M + MX_BM - 1) / MX_BM, nN = (N + MX_BN - 1) / MX_BN;
  int tm, tn;
  xcd_tile(nM, nN, tm, tn);
  const int m0 = tm * MX_BM, n0 = tn * MX_BN;
  const int S = K / MX_KS;
  const uint32_t Kb = static_cast<uint32_t>(K) / 2;     // code bytes per row
  const uint32_t Ks = static_cast<uint32_t>(K) / 32;    // scale bytes per row

  // Loader roles: thread t moves 16-byte chunk (t & 3) of activation rows
  // (t >> 2) + 64 i (i < 2) and of weight rows (t >> 2) + 64 i (i < 4), the
  // scale dword of weight row t and, for t < 128, of activation row t.
  // Buffer resources sized to each operand turn rows past M or N into zeros.
  const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(x_codes), 0, static_cast<int>(static_cast<size_t>(M) * Kb), 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(w_codes), 0, static_cast<int>(static_cast<size_t>(N) * Kb), 0x00020000);
  const __amdgpu_buffer_rsrc_t sa_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(x_scales), 0, static_cast<int>(static_cast<size_t>(M) * Ks), 0x00020000);
  const __amdgpu_buffer_rsrc_t sb_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(w_scales), 0, static_cast<int>(static_cast<size_t>(N) * Ks), 0x00020000);
  const int l_r = tid >> 2, l_c = tid & 3;
  constexpr uint32_t OOB = 0x80000000u;
  uint32_t a_off[2], b_off[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = m0 + l_r + 64 * i;
    a_off[i] = r < M ? static_cast<uint32_t>(r) * Kb + 16u * l_c : OOB;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = n0 + l_r + 64 * i;
    b_off[i] = r < N ? static_cast<uint32_t>(r) * Kb + 16u * l_c : OOB;
  }
  const uint32_t sa_off = (tid < MX_BM && m0 + tid < M) ? static_cast<uint32_t>(m0 + tid) * Ks : OOB;
  const uint32_t sb_off = (n0 + tid < N) ? static_cast<uint32_t>(n0 + tid) * Ks : OOB;

  uint4 ra[2], rb[4];
  uint32_t rsa, rsb;
  auto load_stage = [&](int st) {
    const uint32_t ko = static_cast<uint32_t>(st) * (MX_KS / 2);
    const uint32_t so = static_cast<uint32_t>(st) * (MX_KS / 32);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            a_rs, a_off[i] == OOB ? OOB : a_off[i] + ko, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            b_rs, b_off[i] == OOB ? OOB : b_off[i] + ko, 0, 0));
    rsa = __builtin_amdgcn_raw_buffer_load_b32(sa_rs, sa_off == OOB ? OOB : sa_off + so, 0, 0);
    rsb = __builtin_amdgcn_raw_buffer_load_b32(sb_rs, sb_off == OOB ? OOB : sb_off + so, 0, 0);
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = l_r + 64 * i;
      sm.a[buf][r][mx_swz(r, l_c)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = l_r + 64 * i;
      sm.b[buf][r][mx_swz(r, l_c)] = rb[i];
    }
    if (tid < MX_BM) sm.sa[buf][tid] = rsa;
    sm.sb[buf][tid] = rsb;
  };

  v16f acc[MX_TI][MX_TJ];
#pragma unroll
  for (int i = 0; i < MX_TI; ++i)
#pragma unroll
    for (int j = 0; j < MX_TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int fr = lane & 31;      // fragment row within a 32-row tile
  const int fk = lane >> 5;      // which 32-k block of the k-step

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int st = 0; st < S; ++st) {
    const int buf = st & 1;
    const bool more = (st + 1) < S;
    if (more) load_stage(st + 1);

    uint32_t sxw[MX_TI], sww[MX_TJ];
#pragma unroll
    for (int i = 0; i < MX_TI; ++i) sxw[i] = sm.sa[buf][wm * MX_WM + i * 32 + fr];
#pragma unroll
    for (int j = 0; j < MX_TJ; ++j) sww[j] = sm.sb[buf][wn * MX_WN + j * 32 + fr];
#pragma unroll
    for (int ks = 0; ks < MX_KS / 64; ++ks) {
      const int chunk = 2 * ks + fk;
      v8i xf[MX_TI], wf[MX_TJ];
#pragma unroll
      for (int i = 0; i < MX_TI; ++i) {
        const int r = wm * MX_WM + i * 32 + fr;
        const uint4 u = sm.a[buf][r][mx_swz(r, chunk)];
        xf[i] = v8i{static_cast<int>(u.x), static_cast<int>(u.y), static_cast<int>(u.z), static_cast<int>(u.w),
                    0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < MX_TJ; ++j) {
        const int c = wn * MX_WN + j * 32 + fr;
        const uint4 u = sm.b[buf][c][mx_swz(c, chunk)];
        wf[j] = v8i{static_cast<int>(u.x), static_cast<int>(u.y), static_cast<int>(u.z), static_cast<int>(u.w),
                    0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < MX_TI; ++i) {
        const int sx = static_cast<int>(__builtin_amdgcn_ubfe(sxw[i], 8 * chunk, 8));
#pragma unroll
        for (int j = 0; j < MX_TJ; ++j) {
          const int sw = static_cast<int>(__builtin_amdgcn_ubfe(sww[j], 8 * chunk, 8));
          // cbsz = blgp = 4: both operands FP4 E2M1
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], xf[i], acc[i][j], 4, 4, 0, sw, 0, sx);
        }
      }
    }

    if (more) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: up projection on bf16 MFMA 32x32x16 (K = rank in slices
  // of 16), transposed like the main product.
  const int fk8 = fk;
  if constexpr (HAS_RANK) {
    for (int kk = 0; kk < rank; kk += 16) {
      const int kl = kk + fk8 * 8;
      v8bf la[MX_TI];
#pragma unroll
      for (int i = 0; i < MX_TI; ++i) {
        const int r = m0 + wm * MX_WM + i * 32 + fr;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (r < M) {
          const float4* p = reinterpret_cast<const float4*>(lora_act + static_cast<size_t>(r) * rank + kl);
          const float4 v0 = p[0], v1 = p[1];
          v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
          v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
        }
        la[i] = pack_bf16x8(v);
      }
#pragma unroll
      for (int j = 0; j < MX_TJ; ++j) {
        const int c = n0 + wn * MX_WN + j * 32 + fr;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (c < N) u = *reinterpret_cast<const uint4*>(lora_up + static_cast<size_t>(c) * rank + kl);
        const v8bf ub = __builtin_bit_cast(v8bf, u);
#pragma unroll
        for (int i = 0; i < MX_TI; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ub, la[i], acc[i][j], 0, 0, 0);
      }
    }
  }

  // ---- bias and store.  A lane holds output row m and columns
  // 8b + 4 fk + (0..3) of each 32-column tile.  bf16 output goes through
  // LDS: each wave writes its 64 x 128 tile with 8-byte writes, then stores
  // whole 256-byte row segments, four rows per instruction; 16-byte chunk
  // c of tile row r sits at chunk c ^ (r & 15).
  if (OUT_F32) {
#pragma unroll
    for (int i = 0; i < MX_TI; ++i) {
      const int row = m0 + wm * MX_WM + i * 32 + fr;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < MX_TJ; ++j) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int c = n0 + wn * MX_WN + j * 32 + 8 * bb + 4 * fk;
          if (c >= N) continue;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[i][j][4 * bb + e];
          if (bias) {
            const uint2 bv = *reinterpret_cast<const uint2*>(bias + c);
            o[0] += bf16_bits_to_f32(bv.x & 0xFFFFu);
            o[1] += bf16_bits_to_f32(bv.x >> 16);
            o[2] += bf16_bits_to_f32(bv.y & 0xFFFFu);
            o[3] += bf16_bits_to_f32(bv.y >> 16);
          }
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + static_cast<size_t>(row) * N + c) =
              make_float4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  } else {
    uint2* tile = reinterpret_cast<uint2*>(mx_smem_raw) + wave * (MX_WM * MX_WN / 4);
#pragma unroll
    for (int i = 0; i < MX_TI; ++i) {
      const int rl = i * 32 + fr;
#pragma unroll
      for (int j = 0; j < MX_TJ; ++j) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int c = n0 + wn * MX_WN + j * 32 + 8 * bb + 4 * fk;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[i][j][4 * bb + e];
          if (bias && c < N) {
            const uint2 bv = *reinterpret_cast<const uint2*>(bias + c);
            o[0] += bf16_bits_to_f32(bv.x & 0xFFFFu);
            o[1] += bf16_bits_to_f32(bv.x >> 16);
            o[2] += bf16_bits_to_f32(bv.y & 0xFFFFu);
            o[3] += bf16_bits_to_f32(bv.y >> 16);
          }
          const int chunk = j * 4 + bb;                 // 16-byte chunk of the 256-byte tile row
          tile[rl * 32 + ((chunk ^ (rl & 15)) << 1) + fk] =
              make_uint2(f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16),
                         f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16));
        }
      }
    }
    // the reads below are of another type than the writes above: keep the
    // compiler from moving them across (the hardware orders one wave's LDS ops)
    asm volatile("" ::: "memory");
    const uint4* tile4 = reinterpret_cast<const uint4*>(tile);
    const int cl = lane & 15;                           // 16-byte chunk this lane stores
    const int col = n0 + wn * MX_WN + cl * 8;
#pragma unroll
    for (int it = 0; it < MX_WM / 4; ++it) {
      const int rl = it * 4 + (lane >> 4);
      const uint4 v = tile4[rl * 16 + (cl ^ (rl & 15))];
      const int row = m0 + wm * MX_WM + rl;
      if (row < M && col < N)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(y) + static_cast<size_t>(row) * N + col) = v;
    }
  }
}

template <int OUT_F32, int HAS_RANK>
int launch_mx_kernel(const void* x_codes, const void* x_scales, const void* w_codes, const void* w_scales,
                     const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K,
                     int rank, void* y, hipStream_t st) {
  auto kern = k_gemm_mxfp4_lora_up<OUT_F32, HAS_RANK>;
  static const bool attr_ok = [&] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(MX_SMEM)) == hipSuccess;
  }();
  if (!attr_ok) return SVDQ_ERR_HIP;
  const int nb = ((M + MX_BM - 1) / MX_BM) * ((N + MX_BN - 1) / MX_BN);
  hipLaunchKernelGGL(kern, dim3(nb), dim3(MX_THREADS), MX_SMEM, st, static_cast<const uint8_t*>(x_codes),
                     static_cast<const uint8_t*>(x_scales), static_cast<const uint8_t*>(w_codes),
                     static_cast<const uint8_t*>(w_scales), lora_act, static_cast<const uint16_t*>(lora_up),
                     static_cast<const uint16_t*>(bias), M, N, K, rank, y);
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

}  // namespace

namespace svdq {

int launch_gemm_mxfp4_lora_up(const void* x_codes, const void* x_scales, const void* w_codes,
                              const void* w_scales, const float* lora_act, const void* lora_up,
                              const void* bias, int M, int N, int K, int rank, int out_dtype, void* y,
                              void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (out_dtype == SVDQ_OUT_F32) {
    if (rank > 0)
      return launch_mx_kernel<1, 1>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, st);
    return launch_mx_kernel<1, 0>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, st);
  }
  if (rank > 0)
    return launch_mx_kernel<0, 1>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, st);
  return launch_mx_kernel<0, 0>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, st);
}

}  // namespace svdq
