// HIP kernels for the SVDQuant W4A4 linear on gfx950 (MI355X).
//
// Kernel 1 (k_quant_act_lora_down): smoothing, per-(token, group of 64)
//   symmetric INT4 quantization with nibble packing, and the rank-r down
//   projection X_hat L1 on bf16 MFMA, all from one read of each input element
//   (svdq-int4-flux.1-depth-dev model card, "Nunchaku Engine Design": the
//   quantizer and the down projection share their input).
// Kernel 2 (k_gemm_w4a4_lora_up): INT4 x INT4 GEMM on int8 MFMA with exact
//   int32 per-group products, per-group dequantization, and the up projection
//   (X_hat L1) L2 plus bias in the same fp32 accumulators (same section: the
//   up projection and the 4-bit compute share their output) -- before the K
//   loop in the 256 x 256 form, in the epilogue of the 128 x 128 form.
//
// MFMA operand layouts used (16x16 tiles, wave64):
//   A operand: lane l holds row (l % 16) and one K slice chosen by (l / 16);
//   B operand: lane l holds column (l % 16) and the same K slice;
//   C/D:       lane l holds rows 4*(l/16) + i, i = 0..3, of column (l % 16).
// A and B place K identically, so any permutation of k inside one
// instruction's K range, applied to both operands, leaves the product
// unchanged; the nibble unpacking below relies on that.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq.h"
#include "svdq_internal.h"

#include "svdq_device.h"

namespace {

// =====================================================================
// Kernel 1
// =====================================================================
// QM selects the quantizer: INT4 (group 64, fp16 scale), the same INT4
// codes written as E3M2 values in the 6-bit MFMA fragment layout (FP6; see
// svdq_fp6_kernels.hip), MXFP4 (E2M1 elements, E8M0 scale per 32) or none,
// which leaves only the down projection (the unfused reference path, which
// reads X a second time).
//
// Block: 16 token rows (32 when the 16-row blocks would outnumber the CUs,
// below), 16 waves (8 for ranks above 64, and for a grid larger than the CU
// count: two 8-wave blocks then share a CU instead of leaving a second round
// of blocks); wave w handles
// groups w, w+W, ... of K in batches of up to 2 groups whose loads are all
// issued before any is used, so a CU keeps enough bytes in flight to stream HBM.  smooth_inv is
// staged once per block in LDS.  Lane l works on row (l % 16) and the 16
// consecutive k of its group at offset 16*(l/16); the four lanes of a row
// reduce the group absmax with two cross-lane exchanges.  The down
// projection treats the lane's 16 values as two 16x16x32 bf16 MFMA A
// operands (k offsets 0..7 and 8..15 of its slice); the waves' partial sums
// are reduced through LDS in wave order.
constexpr int K1_ROWS = 16;
constexpr int K1_MAX_WAVES = 16;
// 16 waves per block for ranks up to 64 (4 waves per SIMD hide the load
// latency); 8 waves above, where the down-projection accumulators need the
// registers.
template <int NT> constexpr int k1_waves() { return NT <= 4 ? 16 : 8; }

enum { Q_NONE = 0, Q_INT4 = 1, Q_MXFP4 = 2, Q_FP6 = 3 };

// WB is the largest block the instance is launched with (its register
// budget: 128 VGPRs at 16 waves, 256 at 8).
template <int ACT, int NT, int QM, int RT, int WB>
__global__ __launch_bounds__(WB * 64) void k_quant_act_lora_down(
    const uint16_t* __restrict__ x, const float* __restrict__ smooth_inv,
    const uint16_t* __restrict__ lora_down, int M, int K, int rank,
    uint8_t* __restrict__ x_codes, void* __restrict__ x_scales_v, float* __restrict__ lora_act) {
  extern __shared__ __align__(16) unsigned char k1_smem_raw[];
  float* s_si = reinterpret_cast<float*>(k1_smem_raw);   // [K]
  float* red = s_si + K;                                   // [waves][2][16 RT][16]

  const int nwaves = blockDim.x >> 6;                   // WB or 8 (uniform)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * (K1_ROWS * RT);
  const int kq = (lane >> 4) * 16;
  const int G = K / GROUP;
  const int ntiles = rank >> 4;
  int row[RT];
  bool row_ok[RT];
  const uint16_t* xrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    row[rt] = m0 + K1_ROWS * rt + (lane & 15);
    row_ok[rt] = row[rt] < M;
    xrow[rt] = x + static_cast<size_t>(row_ok[rt] ? row[rt] : 0) * K;
  }

  for (int k = threadIdx.x * 4; k < K; k += blockDim.x * 4)
    *reinterpret_cast<float4*>(s_si + k) = *reinterpret_cast<const float4*>(smooth_inv + k);
  __syncthreads();

  v4f acc[RT][NT > 0 ? NT : 1];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < (NT > 0 ? NT : 1); ++t) acc[rt][t] = v4f{0.f, 0.f, 0.f, 0.f};

  constexpr int K1_BATCH = (NT <= 2 && RT == 1) ? 2 : 1;

  for (int g0 = wave; g0 < G; g0 += nwaves * K1_BATCH) {
    uint4 raw[K1_BATCH][RT][2];
#pragma unroll
    for (int b = 0; b < K1_BATCH; ++b) {
      const int g = g0 + b * nwaves;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        raw[b][rt][0] = raw[b][rt][1] = make_uint4(0, 0, 0, 0);
        if (row_ok[rt] && g < G) {
          raw[b][rt][0] = *reinterpret_cast<const uint4*>(xrow[rt] + g * GROUP + kq);
          raw[b][rt][1] = *reinterpret_cast<const uint4*>(xrow[rt] + g * GROUP + kq + 8);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < K1_BATCH; ++b) {
      const int g = g0 + b * nwaves;
      if (g >= G) break;
      const int k0 = g * GROUP + kq;
      const float4* sp = reinterpret_cast<const float4*>(s_si + k0);
      float4 s4[4] = {sp[0], sp[1], sp[2], sp[3]};
      const float* sv = reinterpret_cast<const float*>(s4);
      v8bf a0[RT], a1[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint32_t w[8] = {raw[b][rt][0].x, raw[b][rt][0].y, raw[b][rt][0].z, raw[b][rt][0].w,
                               raw[b][rt][1].x, raw[b][rt][1].y, raw[b][rt][1].z, raw[b][rt][1].w};
        float xh[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float lo = bf16_bits_to_f32(w[i] & 0xFFFFu);
          float hi = bf16_bits_to_f32(w[i] >> 16);
          if (ACT == SVDQ_ACT_GELU_TANH) {
            lo = gelu_tanh(lo);
            hi = gelu_tanh(hi);
          }
          xh[2 * i] = lo * sv[2 * i];
          xh[2 * i + 1] = hi * sv[2 * i + 1];
        }
        if constexpr (QM == Q_INT4 || QM == Q_FP6) {
          _Float16* x_scales = static_cast<_Float16*>(x_scales_v);
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[i]));
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          const float s32 = amax / 7.0f;
          const _Float16 sh = static_cast<_Float16>(s32);
          const float sf = static_cast<float>(sh);
          const float rcp = (sf == 0.f) ? 0.f : 1.0f / sf;
          if constexpr (QM == Q_INT4) {
            uint32_t p0 = 0, p1 = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float q0 = fminf(fmaxf(rintf(xh[i] * rcp), -8.f), 7.f);
              const float q1 = fminf(fmaxf(rintf(xh[8 + i] * rcp), -8.f), 7.f);
              p0 |= (static_cast<uint32_t>(static_cast<int>(q0)) & 0xFu) << (4 * i);
              p1 |= (static_cast<uint32_t>(static_cast<int>(q1)) & 0xFu) << (4 * i);
            }
            if (row_ok[rt]) {
              *reinterpret_cast<uint2*>(x_codes + static_cast<size_t>(row[rt]) * (K / 2) + (k0 >> 1)) =
                  make_uint2(p0, p1);
              if (lane < 16) x_scales[static_cast<size_t>(g) * M + row[rt]] = sh;
            }
          } else {
            // The lane's 16 codes are codes 16 (q % 2) .. + 15 of fragment
            // lane (row % 32) + 32 (q / 2), q = lane / 16: 96 bits, dwords
            // 0..2 or 3..5 of that lane's string.  The packed conversion
            // puts its first source in the even positions and its second in
            // the odd ones; positions 16..31 are zeros (dwords 3..5 unused).
            // Rows M .. Mp - 1 of the padded last row block are written as
            // zeros (codes +0, scale 0).
            const int RB = (M + 31) >> 5, Mp = RB << 5;
            typedef float v16f_ __attribute__((ext_vector_type(16)));
            v16f_ ev, od;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              // + 0.0f turns -0 into +0 (the codes are integers)
              ev[i] = fminf(fmaxf(rintf(xh[2 * i] * rcp), -8.f), 7.f) + 0.0f;
              od[i] = fminf(fmaxf(rintf(xh[2 * i + 1] * rcp), -8.f), 7.f) + 0.0f;
              ev[8 + i] = 0.f;
              od[8 + i] = 0.f;
            }
            typedef int v6i_ __attribute__((ext_vector_type(6)));
            const v6i_ pk = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, 1.0f);
            if (row[rt] < Mp) {
              const int qq = lane >> 4;
              const int fl = (row[rt] & 31) + 32 * (qq >> 1);
              uint8_t* fr = x_codes + (static_cast<size_t>(g) * RB + (row[rt] >> 5)) * 1536;
              if ((qq & 1) == 0) {
                *reinterpret_cast<uint3*>(fr + 16 * fl) = make_uint3(pk[0], pk[1], pk[2]);
              } else {
                *reinterpret_cast<uint32_t*>(fr + 16 * fl + 12) = static_cast<uint32_t>(pk[0]);
                *reinterpret_cast<uint2*>(fr + 1024 + 8 * fl) = make_uint2(pk[1], pk[2]);
              }
              if (lane < 16) x_scales[static_cast<size_t>(g) * Mp + row[rt]] = sh;
            }
          }
        } else if constexpr (QM == Q_MXFP4) {
          // MXFP4: blocks of 32 k are the lane pairs (l, l ^ 16).  Scale
          // 2^e with e = floor(log2 amax) - 2 read off the exponent field,
          // clamped at -127 (zero and tiny blocks); x_hat * 2^-e is exact.
          uint8_t* x_scales = static_cast<uint8_t*>(x_scales_v);
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[i]));
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          const int ebits = static_cast<int>(__float_as_uint(amax) >> 23);   // amax >= 0
          const int e = max(ebits - 129, -127);
          const float f = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
          // E2M1 code of x_hat * 2^-e: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6,
          // ties to the even code, saturating at 6, +0 for anything that
          // rounds to zero.  gfx950's packed conversion rounds this way
          // (checked on the device over every rounding boundary) except that
          // values rounding to zero from below come out as -0; those are
          // cleared.
          uint32_t p0 = 0, p1 = 0;
          p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, xh[0] * f, xh[1] * f, 1.0f, 0);
          p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, xh[2] * f, xh[3] * f, 1.0f, 1);
          p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, xh[4] * f, xh[5] * f, 1.0f, 2);
          p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, xh[6] * f, xh[7] * f, 1.0f, 3);
          p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, xh[8] * f, xh[9] * f, 1.0f, 0);
          p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, xh[10] * f, xh[11] * f, 1.0f, 1);
          p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, xh[12] * f, xh[13] * f, 1.0f, 2);
          p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, xh[14] * f, xh[15] * f, 1.0f, 3);
          p0 = e2m1_clear_neg_zero(p0);
          p1 = e2m1_clear_neg_zero(p1);
          if (row_ok[rt]) {
            *reinterpret_cast<uint2*>(x_codes + static_cast<size_t>(row[rt]) * (K / 2) + (k0 >> 1)) =
                make_uint2(p0, p1);
            if (((lane >> 4) & 1) == 0)
              x_scales[static_cast<size_t>(row[rt]) * (K / 32) + (k0 >> 5)] = static_cast<uint8_t>(e + 127);
          }
        }
        if constexpr (NT > 0) {
          a0[rt] = pack_bf16x8(xh);
          a1[rt] = pack_bf16x8(xh + 8);
        }
      }
      if constexpr (NT > 0) {
        // each L1 fragment serves every row tile of the block
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < ntiles) {
            const uint16_t* bp = lora_down + static_cast<size_t>(t * 16 + (lane & 15)) * K + k0;
            const v8bf b0 = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(bp));
            const v8bf b1 = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(bp + 8));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[rt], b0, acc[rt][t], 0, 0, 0);
              acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[rt], b1, acc[rt][t], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  if constexpr (NT > 0) {
    // Deterministic cross-wave reduction of the down projection, two rank
    // tiles (32 ranks) at a time, summed in wave order.  red[w][tt][r][c]:
    // wave w's partial of row r (of the block's 16 RT), rank 16 (t0 + tt) + c.
    constexpr int RR = K1_ROWS * RT;
    for (int t0 = 0; t0 < ntiles; t0 += 2) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t == t0 + tt) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                red[((wave * 2 + tt) * RR + K1_ROWS * rt + 4 * (lane >> 4) + i) * 16 + (lane & 15)] = acc[rt][t][i];
          }
        }
      }
      __syncthreads();
      for (int o = threadIdx.x; o < 2 * RR * 16; o += blockDim.x) {
        const int tt = o / (RR * 16);
        const int r = (o >> 4) % RR;
        const int c = o & 15;
        if (t0 + tt < ntiles && m0 + r < M) {
          // in wave order, eight loads in flight at a time (8 or 16 waves)
          float s = 0.f;
          for (int w8 = 0; w8 < nwaves; w8 += 8) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = red[(((w8 + j) * 2 + tt) * RR + r) * 16 + c];
#pragma unroll
            for (int j = 0; j < 8; ++j) s += v[j];
          }
          lora_act[static_cast<size_t>(m0 + r) * rank + (t0 + tt) * 16 + c] = s;
        }
      }
      __syncthreads();
    }
  }
}

// =====================================================================
// Kernel 2
// =====================================================================
// Two tile forms.  The small form (k_gemm_w4a4_lora_up_t128), described
// here, serves odd M and grids with fewer than 192 tiles of 256 x 256; the
// large form further below keeps its arithmetic and changes how operands
// reach LDS.
//
// Block tile 128 x 128, 4 waves in a 2 x 2 arrangement; each wave owns
// 64 x 64 outputs = 4 x 4 tiles of 16 x 16.  Each tile is computed
// transposed, Y^T = W^T X^T: the weight fragment is the MFMA A operand and
// the activation fragment the B operand, so a lane holds one output row and
// runs of four consecutive output columns, which the epilogue stores as
// 8-byte bf16 chunks.  One group of 64 k is one v_mfma_i32_16x16x64_i8 per
// tile.  The K loop runs in stages of two groups: a stage is loaded from HBM
// as packed nibbles into registers one stage ahead, unpacked cooperatively
// (once per block) and written to a double-buffered LDS tile as int8
// operands, so the waves read ready MFMA fragments with one 16-byte LDS read
// each.  Two blocks share a CU, so one block's barrier and load waits
// overlap the other's compute.
//
// 16x16x64 layouts (wave64): A operand lane l holds row l % 16 and the
// 16-k slice l / 16; B operand lane l holds column l % 16 and the same
// slice; C/D lane l holds column l % 16, rows 4 (l / 16) + e in register e.
// Here D rows are output columns n, D columns are output rows m.
//
// Unpacking: a packed dword holds 8 codes (byte j = code 2j low, 2j+1 high).
// (w << 4) & 0xF0F0F0F0 puts the even codes in the high nibble of each byte
// and w & 0xF0F0F0F0 the odd ones, so every int8 lane of the MFMA operand
// equals 16 * q with no sign extension; the product is 256 * P_g.  A and B
// use the same order of k inside the group, which the product ignores.
//
// Dequantization: every group's MFMA takes the constant 0x4B400000 (the bit
// pattern of 1.5 * 2^23) as its C operand.  |256 * P_g| <= 2^20 < 2^22, so
// the int32 result read as fp32 is exactly 1.5 * 2^23 + 256 * P_g.  With
// a = s_x / 256 and b = -1.5 * 2^23 * a (both exact in fp32, kept per output
// row in LDS), fma(D, a, b) = s_x * P_g exactly (11 + 13 significant bits),
// and acc = fma(that, s_w, acc) adds the group with one rounding of
// s_x s_w P_g + acc.  Both are plain fp32 FMAs, which gfx950 issues at twice
// the rate of the mixed-precision form; the weight scales are therefore kept
// as fp32 in LDS (four consecutive columns per 16-byte read).
//
// Schedule: per group the 16 tiles run in a fixed order, and a tile is
// dequantized two tiles after its MFMA was issued (results in a ring of
// four), so the VALU never waits out an MFMA's latency; the second group's
// fragments are read from LDS while the first group computes.  On gfx950 an
// int8 MFMA and fp32 VALU work of the same SIMD do not run concurrently
// (measured: their times add, also with independent operands, at 2 and 4
// waves per SIMD), so the kernel's floor is the MFMA time plus two FMAs per
// output and group.
//
// LDS layout of an unpacked operand row: 64 bytes per group = four 16-byte
// chunks, chunk c holding k slice c (16 codes).  Chunk c of row r is stored
// at position c ^ (((r >> 1) ^ (r >> 3)) & 3), which spreads the loader's
// row-wise writes over the banks; a fragment read (16 consecutive rows, all
// four chunks) covers one contiguous kilobyte either way.
constexpr int K2_BM = 128;
constexpr int K2_BN = 128;
constexpr int K2_SG = 2;                      // groups per pipeline stage
constexpr int K2_WAVES = 4;
constexpr int K2_THREADS = K2_WAVES * 64;
constexpr int K2_WM = 64;                     // wave tile rows (m)
constexpr int K2_WN = 64;                     // wave tile columns (n)
constexpr int K2_TB = K2_WM / 16;             // 16-row activation tiles per wave (m)
constexpr int K2_TA = K2_WN / 16;             // 16-column weight tiles per wave (n)
constexpr int K2_NTILE = K2_TA * K2_TB;
constexpr int MAGIC_I = 0x4B400000;
constexpr float MAGIC_F = 12582912.0f;         // 1.5 * 2^23


struct K2Smem {
  uint4 a[2][K2_SG][K2_BM][4];                 // unpacked activations, 16 B chunks
  uint4 b[2][K2_SG][K2_BN][4];                 // unpacked weights
  float2 xc[2][K2_SG][K2_BM];                  // (s_x / 256, -1.5*2^23 * s_x / 256) per row
  float sw[2][K2_SG][K2_BN];                   // weight scales (fp32) per column
};

__device__ __forceinline__ int k2_swz(int row, int chunk) { return chunk ^ (((row >> 1) ^ (row >> 3)) & 3); }

__device__ __forceinline__ uint4 unpack_lo(uint4 w) {  // codes 0..15 of a 32-code chunk
  return make_uint4((w.x << 4) & 0xF0F0F0F0u, w.x & 0xF0F0F0F0u, (w.y << 4) & 0xF0F0F0F0u, w.y & 0xF0F0F0F0u);
}
__device__ __forceinline__ uint4 unpack_hi(uint4 w) {  // codes 16..31
  return make_uint4((w.z << 4) & 0xF0F0F0F0u, w.z & 0xF0F0F0F0u, (w.w << 4) & 0xF0F0F0F0u, w.w & 0xF0F0F0F0u);
}

// Arguments of the fused QKV epilogue: RMSNorm weights of Q and K heads
// (bf16, 128 each), rotary tables cos / sin [M][64] (NULL: no rotation).
struct QkvArgs {
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos;
  const float* sin;
  float eps;
};
constexpr int QKV_HEAD = 128;

// Epilogue of kernel 2: up projection, bias, fused QKV normalization and
// rotation, store.  acc[a][b][e] holds output row
// m0 + wm*64 + 16b + (lane & 15), column n0 + wn*64 + 16a + 4(lane >> 4) + e.
// All threads of the block call it (the QKV form has a barrier); the LDS
// passed in is free.
template <int OUT_F32, int NT, int EPI>
__device__ __forceinline__ void k2_epilogue(v4f (&acc)[K2_TA][K2_TB], unsigned char* k2_smem_raw, int m0, int n0,
                                            const float* __restrict__ lora_act,
                                            const uint16_t* __restrict__ lora_up,
                                            const uint16_t* __restrict__ bias, int M, int N, int rank,
                                            void* __restrict__ y, const QkvArgs& qa) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lq = lane >> 4;
  // ---- epilogue: up projection (bf16 MFMA 16x16x32, K = rank in slices of
  // 32; ranks are multiples of 16, so the lanes of a slice past the rank
  // contribute zeros), transposed like the main product: lora_up rows are
  // the A operand, lora_act rows the B operand; then the bias.  All loads
  // are unconditional at clamped in-bounds addresses and masked afterwards
  // (loads under per-lane branches would each be waited for in turn).
  uint2 bv[K2_TA];
  if (bias) {                                    // uniform; N % 8 == 0
#pragma unroll
    for (int a = 0; a < K2_TA; ++a)
      bv[a] = *reinterpret_cast<const uint2*>(bias + min(n0 + wn * K2_WN + a * 16 + 4 * lq, N - 4));
  }
  if constexpr (NT > 0) {
    for (int kk = 0; kk < rank; kk += 32) {
      const int kl = kk + lq * 8;          // this lane's 8 k values
      const bool kin = kl < rank;
      const int klc = kin ? kl : 0;
      float4 lv[K2_TB][2];
      uint4 uv[K2_TA];
#pragma unroll
      for (int b = 0; b < K2_TB; ++b) {
        const int r = min(m0 + wm * K2_WM + b * 16 + lr, M - 1);
        const float4* p = reinterpret_cast<const float4*>(lora_act + static_cast<size_t>(r) * rank + klc);
        lv[b][0] = p[0];
        lv[b][1] = p[1];
      }
#pragma unroll
      for (int a = 0; a < K2_TA; ++a) {
        const int c = min(n0 + wn * K2_WN + a * 16 + lr, N - 1);
        uv[a] = *reinterpret_cast<const uint4*>(lora_up + static_cast<size_t>(c) * rank + klc);
      }
      v8bf la[K2_TB];
#pragma unroll
      for (int b = 0; b < K2_TB; ++b) {
        const bool ok = kin && m0 + wm * K2_WM + b * 16 + lr < M;
        const float4 v0 = lv[b][0], v1 = lv[b][1];
        const float v[8] = {ok ? v0.x : 0.f, ok ? v0.y : 0.f, ok ? v0.z : 0.f, ok ? v0.w : 0.f,
                            ok ? v1.x : 0.f, ok ? v1.y : 0.f, ok ? v1.z : 0.f, ok ? v1.w : 0.f};
        la[b] = pack_bf16x8(v);
      }
#pragma unroll
      for (int a = 0; a < K2_TA; ++a) {
        const bool ok = kin && n0 + wn * K2_WN + a * 16 + lr < N;
        const v8bf ub = __builtin_bit_cast(v8bf, ok ? uv[a] : make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int b = 0; b < K2_TB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ub, la[b], acc[a][b], 0, 0, 0);
      }
    }
  }

  // ---- bias, then (fused QKV only) per-head RMSNorm and rotary embedding
  // of the Q and K heads.  A lane holds output rows m0 + wm*64 + 16b + lr
  // and, in each 16-column tile a, columns 16a + 4lq + (0..3).
  if (bias) {
#pragma unroll
    for (int a = 0; a < K2_TA; ++a) {
      if (n0 + wn * K2_WN + a * 16 + 4 * lq >= N) continue;
      const float b4[4] = {bf16_bits_to_f32(bv[a].x & 0xFFFFu), bf16_bits_to_f32(bv[a].x >> 16),
                           bf16_bits_to_f32(bv[a].y & 0xFFFFu), bf16_bits_to_f32(bv[a].y >> 16)};
#pragma unroll
      for (int b = 0; b < K2_TB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[a][b][e] += b4[e];
    }
  }
  if constexpr (EPI == 1) {
    // The block's 128 columns are one head (N = 3 * heads * 128, block tiles
    // aligned to heads).  Q heads come first, then K heads, then V heads,
    // which are left as projected.  This condition is uniform per block.
    const int HD = N / 3;
    if (n0 < 2 * HD) {
      const uint16_t* g = n0 < HD ? qa.gq : qa.gk;
      // sum of squares of each row over the head: this lane's 16 columns,
      // the other three lane quads' 48 (lane ^ 16, lane ^ 32), the other
      // wave's 64 via LDS
      float* red = reinterpret_cast<float*>(k2_smem_raw + K2_WAVES * K2_WM * K2_WN * 2);
#pragma unroll
      for (int b = 0; b < K2_TB; ++b) {
        float t = 0.f;
#pragma unroll
        for (int a = 0; a < K2_TA; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) t = fmaf(acc[a][b][e], acc[a][b][e], t);
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        if (lq == 0) red[((wm * K2_TB + b) * 2 + wn) * 16 + lr] = t;
      }
      // the lane's norm weights (the same for every row), loaded once
      uint2 gv[K2_TA];
#pragma unroll
      for (int a = 0; a < K2_TA; ++a) gv[a] = *reinterpret_cast<const uint2*>(g + wn * K2_WN + a * 16 + 4 * lq);
      const bool rot = qa.cos != nullptr;                 // uniform
      __syncthreads();
#pragma unroll
      for (int b = 0; b < K2_TB; ++b) {
        const float tot = red[((wm * K2_TB + b) * 2 + 0) * 16 + lr] + red[((wm * K2_TB + b) * 2 + 1) * 16 + lr];
        const float scale = 1.0f / sqrtf(tot * (1.0f / QKV_HEAD) + qa.eps);
        // rows past M are never stored: they read row M - 1's factors, so
        // the rotation's loads need no per-lane branch
        const int row = min(m0 + wm * K2_WM + b * 16 + lr, M - 1);
#pragma unroll
        for (int a = 0; a < K2_TA; ++a) {
          const int ch = wn * K2_WN + a * 16 + 4 * lq;        // column within the head
          const float g4[4] = {bf16_bits_to_f32(gv[a].x & 0xFFFFu), bf16_bits_to_f32(gv[a].x >> 16),
                               bf16_bits_to_f32(gv[a].y & 0xFFFFu), bf16_bits_to_f32(gv[a].y >> 16)};
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[a][b][e] * scale * g4[e];
          if (rot) {
            const float2 cs = *reinterpret_cast<const float2*>(qa.cos + static_cast<size_t>(row) * 64 + (ch >> 1));
            const float2 sn = *reinterpret_cast<const float2*>(qa.sin + static_cast<size_t>(row) * 64 + (ch >> 1));
            const float a0 = o[0] * cs.x - o[1] * sn.x, a1 = o[1] * cs.x + o[0] * sn.x;
            const float a2 = o[2] * cs.y - o[3] * sn.y, a3 = o[3] * cs.y + o[2] * sn.y;
            o[0] = a0; o[1] = a1; o[2] = a2; o[3] = a3;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[a][b][e] = o[e];
        }
      }
    }
  }

  // ---- store.  bf16 output goes through LDS (free after the K loop's last
  // barrier): each wave writes its 64 x 64 tile with 8-byte writes, then
  // stores whole 128-byte row segments, eight rows per instruction.
  // 16-byte chunk c of tile row r sits at chunk c ^ (r & 7).
  if (OUT_F32) {
#pragma unroll
    for (int b = 0; b < K2_TB; ++b) {
      const int row = m0 + wm * K2_WM + b * 16 + lr;
      if (row >= M) continue;
#pragma unroll
      for (int a = 0; a < K2_TA; ++a) {
        const int c = n0 + wn * K2_WN + a * 16 + 4 * lq;
        if (c >= N) continue;
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + static_cast<size_t>(row) * N + c) =
            make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
      }
    }
  } else {
    uint2* tile = reinterpret_cast<uint2*>(k2_smem_raw) + wave * (K2_WM * K2_WN / 4);  // 64 x 64 bf16
#pragma unroll
    for (int b = 0; b < K2_TB; ++b) {
      const int rl = b * 16 + lr;
#pragma unroll
      for (int a = 0; a < K2_TA; ++a) {
        const int chunk = 2 * a + (lq >> 1);          // 16-byte chunk of the 128-byte tile row
        tile[rl * 16 + ((chunk ^ (rl & 7)) << 1) + (lq & 1)] =
            make_uint2(bf16x2_bits(acc[a][b][0], acc[a][b][1]),
                       bf16x2_bits(acc[a][b][2], acc[a][b][3]));
      }
    }
    // the reads below are of another type than the writes above: keep the
    // compiler from moving them across (the hardware orders one wave's LDS ops)
    asm volatile("" ::: "memory");
    const uint4* tile4 = reinterpret_cast<const uint4*>(tile);
    const int cl = lane & 7;                            // 16-byte chunk this lane stores
    const int col = n0 + wn * K2_WN + cl * 8;
#pragma unroll
    for (int it = 0; it < K2_WM / 8; ++it) {
      const int rl = it * 8 + (lane >> 3);
      const uint4 v = tile4[rl * 8 + (cl ^ (rl & 7))];
      const int row = m0 + wm * K2_WM + rl;
      if (row < M && col < N)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(y) + static_cast<size_t>(row) * N + col) = v;
    }
  }}

template <int OUT_F32, int NT, int EPI>
__global__ __launch_bounds__(K2_THREADS, 2) void k_gemm_w4a4_lora_up_t128(
    const uint8_t* __restrict__ x_codes, const _Float16* __restrict__ x_scales,
    const uint8_t* __restrict__ w_codes, const _Float16* __restrict__ w_scales,
    const float* __restrict__ lora_act, const uint16_t* __restrict__ lora_up,
    const uint16_t* __restrict__ bias, int M, int N, int K, int rank, void* __restrict__ y, QkvArgs qa) {
  extern __shared__ __align__(16) unsigned char k2_smem_raw[];
  K2Smem& sm = *reinterpret_cast<K2Smem*>(k2_smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int nM = (M + K2_BM - 1) / K2_BM, nN = (N + K2_BN - 1) / K2_BN;
  int tm, tn;
  xcd_tile(nM, nN, tm, tn);
  const int m0 = tm * K2_BM, n0 = tn * K2_BN;
  const int G = K / GROUP;
  const int S = (G + K2_SG - 1) / K2_SG;       // stages
  const size_t Kb = static_cast<size_t>(K) / 2;

  // Loader roles per stage (2 groups): thread t moves both 16-byte halves of
  // the 32 packed bytes of (row t & 127, group (t >> 7) & 1) for the
  // activations and for the weights, plus that row's x scale and that
  // column's w scale.  Loads go through buffer resources sized to the
  // operand, so rows past M or N read as zero; the byte offset is pushed
  // out of range for groups past G (and for the stage after the last), so
  // such a group has zero codes and zero scales and adds exactly zero.
  const int l_r = tid & 127, l_g = (wave >> 1) & 1;
  constexpr uint32_t OOB = 0x80000000u;
  const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(x_codes), 0, static_cast<int>(static_cast<size_t>(M) * Kb), 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(w_codes), 0, static_cast<int>(static_cast<size_t>(N) * Kb), 0x00020000);
  const __amdgpu_buffer_rsrc_t sx_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(x_scales), 0, static_cast<int>(static_cast<size_t>(G) * M * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t sw_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(w_scales), 0, static_cast<int>(static_cast<size_t>(G) * N * 2), 0x00020000);
  // Per-lane byte offsets of stage 0 (2^31 for a scale row past M or N);
  // a stage adds a wave-uniform amount, and a group past G loads from
  // offset 2^31, past every buffer, which returns zeros.
  const uint32_t a_off0 = static_cast<uint32_t>((m0 + l_r) * Kb + l_g * 32);
  const uint32_t b_off0 = static_cast<uint32_t>((n0 + l_r) * Kb + l_g * 32);
  const uint32_t sx_off0 = (m0 + l_r) < M ? static_cast<uint32_t>(2 * (l_g * M + m0 + l_r)) : OOB;
  const uint32_t sw_off0 = (n0 + l_r) < N ? static_cast<uint32_t>(2 * (l_g * N + n0 + l_r)) : OOB;

  uint4 ra0, ra1, rb0, rb1;
  _Float16 rsx, rsw;
  auto load_stage = [&](int st) {
    const bool gok = st * K2_SG + l_g < G;     // wave-uniform
    const uint32_t ko = static_cast<uint32_t>(st) * (K2_SG * 32);
    const uint32_t ao = gok ? a_off0 + ko : OOB, bo = gok ? b_off0 + ko : OOB;
    const uint32_t xo = (gok && sx_off0 != OOB) ? sx_off0 + static_cast<uint32_t>(st) * (2 * K2_SG * M) : OOB;
    const uint32_t wo = (gok && sw_off0 != OOB) ? sw_off0 + static_cast<uint32_t>(st) * (2 * K2_SG * N) : OOB;
    ra0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(a_rs, ao, 0, 0));
    ra1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(a_rs, ao + 16, 0, 0));
    rb0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(b_rs, bo, 0, 0));
    rb1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(b_rs, bo + 16, 0, 0));
    rsx = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(sx_rs, xo, 0, 0));
    rsw = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(sw_rs, wo, 0, 0));
  };
  auto store_stage = [&](int buf) {
    sm.a[buf][l_g][l_r][k2_swz(l_r, 0)] = unpack_lo(ra0);
    sm.a[buf][l_g][l_r][k2_swz(l_r, 1)] = unpack_hi(ra0);
    sm.a[buf][l_g][l_r][k2_swz(l_r, 2)] = unpack_lo(ra1);
    sm.a[buf][l_g][l_r][k2_swz(l_r, 3)] = unpack_hi(ra1);
    sm.b[buf][l_g][l_r][k2_swz(l_r, 0)] = unpack_lo(rb0);
    sm.b[buf][l_g][l_r][k2_swz(l_r, 1)] = unpack_hi(rb0);
    sm.b[buf][l_g][l_r][k2_swz(l_r, 2)] = unpack_lo(rb1);
    sm.b[buf][l_g][l_r][k2_swz(l_r, 3)] = unpack_hi(rb1);
    const float ax = static_cast<float>(rsx) * (1.0f / 256.0f);
    sm.xc[buf][l_g][l_r] = make_float2(ax, -MAGIC_F * ax);
    sm.sw[buf][l_g][l_r] = static_cast<float>(rsw);
  };

  v4f acc[K2_TA][K2_TB];
#pragma unroll
  for (int a = 0; a < K2_TA; ++a)
#pragma unroll
    for (int b = 0; b < K2_TB; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

  v4i cmagic = v4i{MAGIC_I, MAGIC_I, MAGIC_I, MAGIC_I};
  // opaque to the optimizer: kept in 4 VGPRs instead of being rebuilt from
  // scalar constants before every MFMA that reads it
  asm volatile("" : "+v"(cmagic));
  const int lr = lane & 15;      // fragment row / output column within a 16-tile
  const int lq = lane >> 4;      // k slice / output row quad

  // Fragments and scales of one group, read from LDS: the lane's weight
  // rows (n) wn*64 + 16a + lr, activation rows (m) wm*64 + 16b + lr, the
  // activation scale pairs of those rows and the weight scales of the four
  // output columns 16a + 4lq .. +3 it accumulates.
  struct Frags {
    v4i w[K2_TA];
    v4i x[K2_TB];
    float2 xc[K2_TB];
    float4 sw[K2_TA];
  };
  auto read_frags = [&](int buf, int gi, Frags& f) {
#pragma unroll
    for (int a = 0; a < K2_TA; ++a) {
      const int c = wn * K2_WN + a * 16 + lr;
      f.w[a] = __builtin_bit_cast(v4i, sm.b[buf][gi][c][k2_swz(c, lq)]);
    }
#pragma unroll
    for (int b = 0; b < K2_TB; ++b) {
      const int r = wm * K2_WM + b * 16 + lr;
      f.x[b] = __builtin_bit_cast(v4i, sm.a[buf][gi][r][k2_swz(r, lq)]);
    }
#pragma unroll
    for (int b = 0; b < K2_TB; ++b) f.xc[b] = sm.xc[buf][gi][wm * K2_WM + b * 16 + lr];
#pragma unroll
    for (int a = 0; a < K2_TA; ++a)
      f.sw[a] = *reinterpret_cast<const float4*>(&sm.sw[buf][gi][wn * K2_WN + a * 16 + 4 * lq]);
  };
  // acc += s_w * (s_x * P): two fp32 FMAs per output
  auto deq = [&](float2 xc, float4 sw, const v4i& d, v4f& ac) {
    const float s4[4] = {sw.x, sw.y, sw.z, sw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float tv = __builtin_fmaf(__int_as_float(d[e]), xc.x, xc.y);
      ac[e] = __builtin_fmaf(tv, s4[e], ac[e]);
    }
  };

  load_stage(0);
  store_stage(0);
  __syncthreads();

  static_assert(K2_SG == 2, "the stage body below holds two groups");
  // Tiles t = 0 .. 31 of a stage (group t / 16, weight tile (t % 16) / 4,
  // activation tile t % 4): the MFMA of tile t is issued, then tile t - 2 is
  // dequantized; results rotate through a ring of four, so the last two
  // tiles of a stage are dequantized at the start of the next one, after
  // the barrier, while the new fragments are still in flight.  Before the
  // first stage the pending tiles are zero contributions (scale pair 0, 0
  // maps the magic constant to exactly 0).
  constexpr int LAG = 2, RING = 4;
  static_assert((2 * K2_NTILE) % RING == 0, "ring slots repeat per stage");
  Frags f0, f1;
  read_frags(0, 0, f0);
#pragma unroll
  for (int b = 0; b < K2_TB; ++b) f1.xc[b] = make_float2(0.f, 0.f);
#pragma unroll
  for (int a = 0; a < K2_TA; ++a) f1.sw[a] = make_float4(0.f, 0.f, 0.f, 0.f);
  v4i dr[RING];
#pragma unroll
  for (int i = 0; i < RING; ++i) dr[i] = cmagic;
  auto deq_tile = [&](int q) {                 // q in 0 .. 31 of the stage whose fragments f0 / f1 hold
    const int u = q % K2_NTILE, a = u / K2_TB, b = u % K2_TB;
    const Frags& f = q < K2_NTILE ? f0 : f1;
    deq(f.xc[b], f.sw[a], dr[q % RING], acc[a][b]);
  };
  for (int st = 0; st < S; ++st) {
    const int buf = st & 1;
    load_stage(st + 1);
#pragma unroll
    for (int t = 0; t < 2 * K2_NTILE; ++t) {
      const int u = t % K2_NTILE, a = u / K2_TB, b = u % K2_TB;
      const Frags& f = t < K2_NTILE ? f0 : f1;
      dr[t % RING] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.w[a], f.x[b], cmagic, 0, 0, 0);
      deq_tile(t >= LAG ? t - LAG : 2 * K2_NTILE - LAG + t);   // t < LAG: the previous stage's last tiles
      if (t == LAG) read_frags(buf, 1, f1);
    }
    store_stage(buf ^ 1);
    __syncthreads();
    read_frags(buf ^ 1, 0, f0);
  }
#pragma unroll
  for (int q = 2 * K2_NTILE - LAG; q < 2 * K2_NTILE; ++q) deq_tile(q);

  k2_epilogue<OUT_F32, NT, EPI>(acc, k2_smem_raw, m0, n0, lora_act, lora_up, bias, M, N, rank, y, qa);
}

// ---------------------------------------------------------------------
// Kernel 2, large form: block tile 256 (m) x 256 (n), 8 waves in a 4 x 2
// grid, each owning 64 (m) x 128 (n) outputs = 4 x 8 tiles of 16 x 16
// computed transposed as above.  A wave's 128 columns are one head of the
// fused QKV layout, so its per-head normalization stays inside the wave.
//
// Operands are not staged through registers: packed codes and the raw fp16
// scales move from HBM straight into a ring of KT_NS LDS stage buffers with
// LDS-DMA buffer loads (no registers, no unpack pass), and each lane unpacks
// the 8 packed bytes of its own fragment when it reads them (three ALU ops
// per packed dword).  Stage = two groups (128 k).  At the top of stage u the
// loads of stage u + 1 have landed as well; during stage u every thread
// converts two of stage u + 1's scales in place to fp32 (s_x / 256 for the
// activations, s_w for the weights), which the next barrier publishes, so
// the only vector-memory operations in the loop are the DMA loads, counted
// exactly by the explicit s_waitcnt.
//
// Stage layout (bytes): activation codes [256 rows][64], weight codes
// [256 rows][64] (16-byte chunk c = group c / 2, packed bytes 16 (c % 2) ..
// + 15 of that group, at position c ^ swz(row)), then one dword per scale:
// activations [2 groups][256], weights [2 groups][256].  A raw scale dword
// is the aligned pair holding the scale (x_scales and w_scales are read as
// pairs, so M must be even here; N is a multiple of 8).
constexpr int KT_BM = 256;
constexpr int KT_BN = 256;
constexpr int KT_WAVES = 8;
constexpr int KT_THREADS = KT_WAVES * 64;
constexpr int KT_WM = 64;
constexpr int KT_WN = 128;
constexpr int KT_TB = KT_WM / 16;             // activation fragments per wave (m)
constexpr int KT_TA = KT_WN / 16;             // weight fragments per wave (n)
constexpr int KT_NS = 4;                      // ring depth (stages)
constexpr int KT_X_BYTES = KT_BM * 64;
constexpr int KT_W_BYTES = KT_BN * 64;
constexpr int KT_SX_OFF = KT_X_BYTES + KT_W_BYTES;
constexpr int KT_SW_OFF = KT_SX_OFF + 2 * KT_BM * 4;
constexpr int KT_STAGE = KT_SW_OFF + 2 * KT_BN * 4;
constexpr int KT_X_INSTR = KT_BM / 16 / KT_WAVES;                      // 1 KB code loads per wave
constexpr int KT_W_INSTR = KT_BN / 16 / KT_WAVES;
constexpr int KT_S_INSTR = (2 * KT_BM / 64 + 2 * KT_BN / 64) / KT_WAVES;  // 256-byte scale loads
constexpr int KT_P = KT_X_INSTR + KT_W_INSTR + KT_S_INSTR;             // DMA loads per wave per stage
static_assert(KT_S_INSTR * KT_WAVES == 2 * KT_BM / 64 + 2 * KT_BN / 64, "equal DMA counts per wave");
static_assert(KT_STAGE % 16 == 0, "stage buffers stay 16-byte aligned");
static_assert(KT_WAVES * KT_WM * KT_WN * 2 <= KT_NS * KT_STAGE, "the output tiles reuse the stage ring");
static_assert(2 * (KT_BM + KT_BN) == 2 * KT_THREADS, "two scale conversions per thread per stage");

// Start values of the large form's accumulators: bias, then the up
// projection (X_hat L1) L2 on bf16 MFMA.  acc[a][b][e] is output row m0 +
// 64 wm + 16b + (lane & 15), column n0 + 128 wn + 16a + 4(lane >> 4) + e.
// The loads of the first 32 ranks and of the bias are issued before the
// first stages' DMA (kt_init_load) and consumed after it (kt_init_acc), so
// that their latency overlaps those loads.  Every load is unconditional at
// a clamped in-bounds address and masked afterwards: loads under per-lane
// branches would each be waited for before the next is issued.
struct KtInit {
  uint2 bv[KT_TA];           // bias, columns 16a + 4lq .. + 3
  float4 la[KT_TB][2];       // lora_act, row 16b + lr, ranks 8lq .. + 7 of the slice
  uint4 lu[KT_TA];           // lora_up, row (output column) 16a + lr, same ranks
};

template <int NT>
__device__ __forceinline__ void kt_init_rank_loads(KtInit& R, int kk, int mw, int nw, const float* __restrict__ lora_act,
                                                   const uint16_t* __restrict__ lora_up, int M, int N, int rank) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int kl = kk + lq * 8;
  const int klc = kl < rank ? kl : 0;
#pragma unroll
  for (int b = 0; b < KT_TB; ++b) {
    const int r = min(mw + b * 16 + lr, M - 1);
    const float4* p = reinterpret_cast<const float4*>(lora_act + static_cast<size_t>(r) * rank + klc);
    R.la[b][0] = p[0];
    R.la[b][1] = p[1];
  }
#pragma unroll
  for (int a = 0; a < KT_TA; ++a) {
    const int c = min(nw + a * 16 + lr, N - 1);
    R.lu[a] = *reinterpret_cast<const uint4*>(lora_up + static_cast<size_t>(c) * rank + klc);
  }
}

template <int NT>
__device__ __forceinline__ void kt_init_load(KtInit& R, int m0, int n0, const float* __restrict__ lora_act,
                                             const uint16_t* __restrict__ lora_up,
                                             const uint16_t* __restrict__ bias, int M, int N, int rank) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lq = lane >> 4;
  const int mw = m0 + wm * KT_WM, nw = n0 + wn * KT_WN;
  if (bias) {                                   // uniform
#pragma unroll
    for (int a = 0; a < KT_TA; ++a)             // N % 8 == 0: four columns all in or all out
      R.bv[a] = *reinterpret_cast<const uint2*>(bias + min(nw + a * 16 + 4 * lq, N - 4));
  }
  if constexpr (NT > 0) kt_init_rank_loads<NT>(R, 0, mw, nw, lora_act, lora_up, M, N, rank);
}

template <int NT>
__device__ __forceinline__ void kt_init_acc(v4f (&acc)[KT_TA][KT_TB], KtInit& R, int m0, int n0,
                                            const float* __restrict__ lora_act,
                                            const uint16_t* __restrict__ lora_up,
                                            const uint16_t* __restrict__ bias, int M, int N, int rank) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lq = lane >> 4;
  const int mw = m0 + wm * KT_WM, nw = n0 + wn * KT_WN;
#pragma unroll
  for (int a = 0; a < KT_TA; ++a) {
    float b4[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias && nw + a * 16 + 4 * lq < N) {
      b4[0] = bf16_bits_to_f32(R.bv[a].x & 0xFFFFu);
      b4[1] = bf16_bits_to_f32(R.bv[a].x >> 16);
      b4[2] = bf16_bits_to_f32(R.bv[a].y & 0xFFFFu);
      b4[3] = bf16_bits_to_f32(R.bv[a].y >> 16);
    }
#pragma unroll
    for (int b = 0; b < KT_TB; ++b) acc[a][b] = v4f{b4[0], b4[1], b4[2], b4[3]};
  }
  // up projection: bf16 MFMA 16x16x32 over the rank in slices of 32 (ranks
  // are multiples of 16, so the lanes of a slice past the rank contribute
  // zeros); lora_up rows are the A operand, lora_act rows the B operand
  if constexpr (NT > 0) {
    for (int kk = 0; kk < rank; kk += 32) {
      if (kk > 0) kt_init_rank_loads<NT>(R, kk, mw, nw, lora_act, lora_up, M, N, rank);
      const bool kin = kk + lq * 8 < rank;
      v8bf la[KT_TB];
#pragma unroll
      for (int b = 0; b < KT_TB; ++b) {
        const bool ok = kin && mw + b * 16 + lr < M;
        const float4 v0 = R.la[b][0], v1 = R.la[b][1];
        const float v[8] = {ok ? v0.x : 0.f, ok ? v0.y : 0.f, ok ? v0.z : 0.f, ok ? v0.w : 0.f,
                            ok ? v1.x : 0.f, ok ? v1.y : 0.f, ok ? v1.z : 0.f, ok ? v1.w : 0.f};
        la[b] = pack_bf16x8(v);
      }
#pragma unroll
      for (int a = 0; a < KT_TA; ++a) {
        const bool ok = kin && nw + a * 16 + lr < N;
        const uint4 u = ok ? R.lu[a] : make_uint4(0, 0, 0, 0);
        const v8bf ub = __builtin_bit_cast(v8bf, u);
#pragma unroll
        for (int b = 0; b < KT_TB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ub, la[b], acc[a][b], 0, 0, 0);
      }
    }
  }
}

// Epilogue of the large form: fused QKV normalization and rotation, store
// (bias and the up projection are already in the accumulators).  acc[a][b][e] holds output row m0 + 64 wm + 16b +
// (lane & 15), column n0 + 128 wn + 16a + 4(lane >> 4) + e.  The LDS passed
// in is free.
template <int OUT_F32, int EPI>
__device__ __forceinline__ void kt_epilogue(v4f (&acc)[KT_TA][KT_TB], unsigned char* smem, int m0, int n0,
                                            int M, int N, void* __restrict__ y, const QkvArgs& qa) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lq = lane >> 4;
  const int mw = m0 + wm * KT_WM, nw = n0 + wn * KT_WN;
  if constexpr (EPI == 1) {
    // The wave's 128 columns are one head (N = 3 * heads * 128): Q heads,
    // then K heads, then V heads, which are left as projected.
    const int HD = N / 3;
    const bool rot = qa.cos != nullptr;                        // uniform
    // The rotary factors of the block's 256 rows go to LDS by LDS-DMA (no
    // registers; the accumulators hold most of them): 16-byte chunk c of row
    // r sits at chunk c ^ (r & 15) of its 256-byte row, which keeps the
    // per-lane reads below free of bank conflicts.  A DMA load of a wave
    // fills four rows: lane l lands at row l / 16, position l % 16, and so
    // fetches chunk (l % 16) ^ (row & 15).  Rows past M read zeros (never
    // stored).  Blocks whose columns are all V skip it.
    float4* lcs = reinterpret_cast<float4*>(smem);              // [256][16] cos
    float4* lsn = lcs + KT_BM * 16;                             // [256][16] sin
    const bool stage = rot && n0 < 2 * HD;                      // uniform per block
    if (stage) {
      constexpr int Q = KT_BM / 4 / KT_WAVES;                   // DMA loads per wave per table
      const uint32_t tbytes = static_cast<uint32_t>(M) * 256u;
      const DmaRsrc crs = dma_rsrc(qa.cos, tbytes), srs = dma_rsrc(qa.sin, tbytes);
      const uint32_t l0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
#pragma unroll
      for (int j = 0; j < Q; ++j) {
        const int q = wave * Q + j;
        const int r = 4 * q + (lane >> 4);
        const uint32_t voff = m0 + r < M ? static_cast<uint32_t>(m0 + r) * 256u + 16u * ((lane & 15) ^ (r & 15))
                                         : 0x80000000u;
        const uint32_t la = __builtin_amdgcn_readfirstlane(l0 + 1024u * q);
        dma16(crs, la, voff);
        dma16(srs, la + KT_BM * 256u, voff);
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      __syncthreads();
    }
    if (nw < 2 * HD) {
      const uint16_t* g = nw < HD ? qa.gq : qa.gk;
      // the lane's norm weights (columns 16a + 4lq .. + 3 of the head, the
      // same for every row), loaded once
      uint2 gv[KT_TA];
#pragma unroll
      for (int a = 0; a < KT_TA; ++a) gv[a] = *reinterpret_cast<const uint2*>(g + a * 16 + 4 * lq);
#pragma unroll
      for (int b = 0; b < KT_TB; ++b) {
        // sum of squares of the row over the head: this lane's 32 columns
        // and the other three lane quads' (lane ^ 16, lane ^ 32)
        float t = 0.f;
#pragma unroll
        for (int a = 0; a < KT_TA; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) t = fmaf(acc[a][b][e], acc[a][b][e], t);
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        const float scale = 1.0f / sqrtf(t * (1.0f / QKV_HEAD) + qa.eps);
        const int rl = wm * KT_WM + b * 16 + lr;               // row within the block
#pragma unroll
        for (int a = 0; a < KT_TA; ++a) {
          const float g4[4] = {bf16_bits_to_f32(gv[a].x & 0xFFFFu), bf16_bits_to_f32(gv[a].x >> 16),
                               bf16_bits_to_f32(gv[a].y & 0xFFFFu), bf16_bits_to_f32(gv[a].y >> 16)};
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[a][b][e] * scale * g4[e];
          if (rot) {
            // columns 16a + 4lq .. + 3 rotate by factors 8a + 2lq and + 1:
            // chunk 2a + lq / 2 of the row, half lq % 2
            const int pos = rl * 16 + ((2 * a + (lq >> 1)) ^ (rl & 15));
            const float2 cs = reinterpret_cast<const float2*>(lcs + pos)[lq & 1];
            const float2 sn = reinterpret_cast<const float2*>(lsn + pos)[lq & 1];
            const float a0 = o[0] * cs.x - o[1] * sn.x, a1 = o[1] * cs.x + o[0] * sn.x;
            const float a2 = o[2] * cs.y - o[3] * sn.y, a3 = o[3] * cs.y + o[2] * sn.y;
            o[0] = a0; o[1] = a1; o[2] = a2; o[3] = a3;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[a][b][e] = o[e];
        }
      }
    }
    if (stage && !OUT_F32) __syncthreads();                     // the output tiles below reuse this LDS
  }
  if (OUT_F32) {
#pragma unroll
    for (int b = 0; b < KT_TB; ++b) {
      const int row = mw + b * 16 + lr;
      if (row >= M) continue;
#pragma unroll
      for (int a = 0; a < KT_TA; ++a) {
        const int c = nw + a * 16 + 4 * lq;
        if (c >= N) continue;
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + static_cast<size_t>(row) * N + c) =
            make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
      }
    }
  } else {
    // bf16 through LDS: each wave writes its 64 x 128 tile with 8-byte
    // writes, then stores whole 256-byte row segments, four rows per
    // instruction; 16-byte chunk c of tile row r sits at chunk c ^ (r & 15).
    uint2* tile = reinterpret_cast<uint2*>(smem) + wave * (KT_WM * KT_WN / 4);
#pragma unroll
    for (int b = 0; b < KT_TB; ++b) {
      const int rl = b * 16 + lr;
#pragma unroll
      for (int a = 0; a < KT_TA; ++a) {
        const int chunk = 2 * a + (lq >> 1);
        tile[rl * 32 + ((chunk ^ (rl & 15)) << 1) + (lq & 1)] =
            make_uint2(bf16x2_bits(acc[a][b][0], acc[a][b][1]),
                       bf16x2_bits(acc[a][b][2], acc[a][b][3]));
      }
    }
    // the reads below are of another type than the writes above: keep the
    // compiler from moving them across (the hardware orders one wave's LDS ops)
    asm volatile("" ::: "memory");
    const uint4* tile4 = reinterpret_cast<const uint4*>(tile);
    const int cl = lane & 15;
    const int col = nw + cl * 8;
#pragma unroll
    for (int it = 0; it < KT_WM / 4; ++it) {
      const int rl = it * 4 + (lane >> 4);
      const uint4 v = tile4[rl * 16 + (cl ^ (rl & 15))];
      const int row = mw + rl;
      if (row < M && col < N)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(y) + static_cast<size_t>(row) * N + col) = v;
    }
  }
}

__device__ __forceinline__ v4i unpack_b64(uint2 w) {   // 16 packed codes -> 16 int8 lanes of 16q
  return v4i{static_cast<int>((w.x << 4) & 0xF0F0F0F0u), static_cast<int>(w.x & 0xF0F0F0F0u),
             static_cast<int>((w.y << 4) & 0xF0F0F0F0u), static_cast<int>(w.y & 0xF0F0F0F0u)};
}

template <int OUT_F32, int NT, int EPI>
__global__ __launch_bounds__(KT_THREADS, 1) void k_gemm_w4a4_lora_up(
    const uint8_t* __restrict__ x_codes, const _Float16* __restrict__ x_scales,
    const uint8_t* __restrict__ w_codes, const _Float16* __restrict__ w_scales,
    const float* __restrict__ lora_act, const uint16_t* __restrict__ lora_up,
    const uint16_t* __restrict__ bias, int M, int N, int K, int rank, void* __restrict__ y, QkvArgs qa) {
  // statically sized ring: with the slot as the first index the compiler
  // can tell the slots apart
  __shared__ __align__(16) unsigned char ring[KT_NS][KT_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nM = (M + KT_BM - 1) / KT_BM, nN = (N + KT_BN - 1) / KT_BN;
  int tm, tn;
  xcd_tile(nM, nN, tm, tn);
  const int m0 = tm * KT_BM, n0 = tn * KT_BN;
  const int G = K / GROUP;
  const int S = (G + 1) / 2;
  const uint32_t Kb = static_cast<uint32_t>(K) / 2;
  constexpr uint32_t OOB = 0x80000000u;

  const DmaRsrc x_rs = dma_rsrc(x_codes, static_cast<uint32_t>(static_cast<size_t>(M) * Kb));
  const DmaRsrc w_rs = dma_rsrc(w_codes, static_cast<uint32_t>(static_cast<size_t>(N) * Kb));
  const DmaRsrc sx_rs = dma_rsrc(x_scales, static_cast<uint32_t>(static_cast<size_t>(G) * M * 2));
  const DmaRsrc sw_rs = dma_rsrc(w_scales, static_cast<uint32_t>(static_cast<size_t>(G) * N * 2));

  // DMA roles.  Code load i of this wave covers 16 rows (1 KB): lane l
  // fetches row 16q + l / 4, logical chunk (l & 3) ^ swz(row), landing at
  // position l & 3; a chunk of a group past G, or a row past M / N, reads as
  // zero.  Scale load j covers 64 consecutive rows of one group and operand:
  // lane l fetches the aligned dword holding that row's fp16 scale.
  uint32_t x_off[KT_X_INSTR], w_off[KT_W_INSTR], s_off[KT_S_INSTR], s_step[KT_S_INSTR];
  int x_grp[KT_X_INSTR], w_grp[KT_W_INSTR], s_grp[KT_S_INSTR];
  bool s_is_x[KT_S_INSTR];
  uint32_t x_lds[KT_X_INSTR], w_lds[KT_W_INSTR], s_lds[KT_S_INSTR];
  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[0][0]));
#pragma unroll
  for (int i = 0; i < KT_X_INSTR; ++i) {
    const int q = wave * KT_X_INSTR + i;
    const int r = 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ k2_swz(r, 0);
    x_off[i] = (m0 + r < M) ? static_cast<uint32_t>(m0 + r) * Kb + 16u * c : OOB;
    x_grp[i] = c >> 1;
    x_lds[i] = __builtin_amdgcn_readfirstlane(ring0 + 1024 * q);
  }
#pragma unroll
  for (int i = 0; i < KT_W_INSTR; ++i) {
    const int q = wave * KT_W_INSTR + i;
    const int r = 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ k2_swz(r, 0);
    w_off[i] = (n0 + r < N) ? static_cast<uint32_t>(n0 + r) * Kb + 16u * c : OOB;
    w_grp[i] = c >> 1;
    w_lds[i] = __builtin_amdgcn_readfirstlane(ring0 + KT_X_BYTES + 1024 * q);
  }
#pragma unroll
  for (int i = 0; i < KT_S_INSTR; ++i) {
    const int j = wave * KT_S_INSTR + i;                       // wave-uniform
    const bool isx = j < 2 * KT_BM / 64;
    const int jj = isx ? j : j - 2 * KT_BM / 64;
    const int gi = jj >> 2, ch = jj & 3;                       // 4 loads of 64 rows per group
    const int r = 64 * ch + lane;
    const int base = isx ? m0 : n0, lim = isx ? M : N;
    const uint32_t e0 = static_cast<uint32_t>(gi) * static_cast<uint32_t>(lim) + static_cast<uint32_t>(base + r);
    s_is_x[i] = isx;
    s_grp[i] = gi;
    s_off[i] = (base + r < lim) ? 4u * (e0 >> 1) : OOB;
    s_step[i] = 4u * static_cast<uint32_t>(lim);               // two groups = 2 * lim scales further
    s_lds[i] = __builtin_amdgcn_readfirstlane(ring0 + (isx ? KT_SX_OFF : KT_SW_OFF) + 4 * (gi * 256 + 64 * ch));
  }

  // Issue the DMA loads of stage st into ring slot `slot` = st % KT_NS.
  auto issue_stage = [&](int st, int slot) {
    const uint32_t so = static_cast<uint32_t>(slot) * KT_STAGE;
    const bool live = st < S;
    const uint32_t ko = static_cast<uint32_t>(st) * 64u;
#pragma unroll
    for (int i = 0; i < KT_X_INSTR; ++i) {
      const bool ok = live && x_off[i] != OOB && 2 * st + x_grp[i] < G;
      dma16(x_rs, x_lds[i] + so, ok ? x_off[i] + ko : OOB);
    }
#pragma unroll
    for (int i = 0; i < KT_W_INSTR; ++i) {
      const bool ok = live && w_off[i] != OOB && 2 * st + w_grp[i] < G;
      dma16(w_rs, w_lds[i] + so, ok ? w_off[i] + ko : OOB);
    }
#pragma unroll
    for (int i = 0; i < KT_S_INSTR; ++i) {
      const bool ok = live && s_off[i] != OOB && 2 * st + s_grp[i] < G;
      dma4(s_is_x[i] ? sx_rs : sw_rs, s_lds[i] + so, ok ? s_off[i] + static_cast<uint32_t>(st) * s_step[i] : OOB);
    }
  };
  // Convert the raw scale dwords of a landed stage to fp32 in place: thread
  // t owns activation scale t (group t / 256, row t % 256) and weight scale
  // t; the fp16 value is the half (row & 1) of its dword (M, N, m0 and n0
  // even).
  auto convert_stage = [&](int slot) {
    uint32_t* sc = reinterpret_cast<uint32_t*>(&ring[slot][KT_SX_OFF]);
    const uint32_t dx = sc[tid], dw = sc[KT_THREADS + tid];
    const int sh = 16 * (tid & 1);
    const float fx = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(dx >> sh)));
    const float fw = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(dw >> sh)));
    sc[tid] = __float_as_uint(fx * (1.0f / 256.0f));
    sc[KT_THREADS + tid] = __float_as_uint(fw);
  };

  v4f acc[KT_TA][KT_TB];
  v4i cmagic = v4i{MAGIC_I, MAGIC_I, MAGIC_I, MAGIC_I};
  asm volatile("" : "+v"(cmagic));

  const int lr = lane & 15, lq = lane >> 4;
  // Per-lane byte offsets in a stage of this lane's fragment reads: the 8
  // packed bytes 8 lq .. 8 lq + 7 of group gi of row r sit in logical chunk
  // 2 gi + lq / 2 at byte 8 (lq & 1).  swz(r) depends on the row bits 1..4,
  // so rows 32 apart share it: one offset per (group, tile parity).
  uint32_t fx_off[2][2], fw_off[2][2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int rx = wm * KT_WM + 16 * p + lr, rw = wn * KT_WN + 16 * p + lr;
      fx_off[gi][p] = rx * 64 + 16 * ((2 * gi + (lq >> 1)) ^ k2_swz(rx, 0)) + 8 * (lq & 1);
      fw_off[gi][p] = KT_X_BYTES + rw * 64 + 16 * ((2 * gi + (lq >> 1)) ^ k2_swz(rw, 0)) + 8 * (lq & 1);
    }
  const uint32_t xs_off = KT_SX_OFF + 4 * (wm * KT_WM + lr);
  const uint32_t ws_off = KT_SW_OFF + 4 * (wn * KT_WN + 4 * lq);

  v4i fx[KT_TB], fw[2];
  float2 xc[2][KT_TB];
  float4 swr[4];
  v4i dr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dr[i] = cmagic;
    swr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int b = 0; b < KT_TB; ++b) xc[0][b] = xc[1][b] = make_float2(0.f, 0.f);

  // Packed code fragments of a stage's first group (activation fragments
  // 0 .. 3 and weight fragment 0), read before the barrier that opens it.
  uint2 px[KT_TB], pw;
  auto rd_first_codes = [&](const unsigned char* s) {
#pragma unroll
    for (int b = 0; b < KT_TB; ++b) px[b] = *reinterpret_cast<const uint2*>(s + fx_off[0][b & 1] + (b >> 1) * 2048);
    pw = *reinterpret_cast<const uint2*>(s + fw_off[0][0]);
  };
  auto rd_w = [&](const unsigned char* s, int gi, int a, v4i& f, float4& sw) {
    f = unpack_b64(*reinterpret_cast<const uint2*>(s + fw_off[gi][a & 1] + (a >> 1) * 2048));
    sw = *reinterpret_cast<const float4*>(s + ws_off + gi * 1024 + 64 * a);
  };
  // acc += s_w * (s_x * P): two fp32 FMAs per output (see the 128 x 128 form)
  auto deq = [&](float2 c, float4 sw, const v4i& d, v4f& ac) {
    const float s4[4] = {sw.x, sw.y, sw.z, sw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) ac[e] = __builtin_fmaf(__builtin_fmaf(__int_as_float(d[e]), c.x, c.y), s4[e], ac[e]);
  };
  // tile q of a stage (0 .. 63): group q / 32, weight fragment (q / 4) % 8,
  // activation fragment q % 4
  auto deq_tile = [&](int q) {
    const int gi = q >> 5, a = (q >> 2) & 7, b = q & 3;
    deq(xc[gi][b], swr[a & 3], dr[q & 3], acc[a][b]);
  };

  // bias and up-projection operands requested, then stages 0 .. 2; the
  // accumulators start while the stages load; stage 0 landed and its
  // scales converted
  KtInit init;
  kt_init_load<NT>(init, m0, n0, lora_act, lora_up, bias, M, N, rank);
#pragma unroll
  for (int st = 0; st < KT_NS - 1; ++st) issue_stage(st, st);
  kt_init_acc<NT>(acc, init, m0, n0, lora_act, lora_up, bias, M, N, rank);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(KT_P * (KT_NS - 2)));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  convert_stage(0);
  rd_first_codes(ring[0]);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(KT_P * (KT_NS - 2)));

  for (int u = 0; u < S; ++u) {
    // stage u + 1 has landed once one stage of this wave's loads is still
    // outstanding; the barrier publishes it with stage u's fp32 scales and
    // frees slot (u - 1) % KT_NS, which every wave has finished reading.
    // LDS operations need no wait here: the scale writes of the previous
    // stage's conversion precede reads that were waited for, and the code
    // fragments read for this stage may still be in flight.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(KT_P * (KT_NS - 3)));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_stage(u + KT_NS - 1, (u + KT_NS - 1) % KT_NS);
    convert_stage((u + 1) % KT_NS);

    const unsigned char* s = ring[u % KT_NS];
#pragma unroll
    for (int b = 0; b < KT_TB; ++b) {
      fx[b] = unpack_b64(px[b]);
      const float ax = *reinterpret_cast<const float*>(s + xs_off + 64 * b);
      xc[0][b] = make_float2(ax, -MAGIC_F * ax);
    }
    fw[0] = unpack_b64(pw);
    swr[0] = *reinterpret_cast<const float4*>(s + ws_off);
    // Tile t: the MFMA of t is issued, then tile t - 2 is dequantized (the
    // two last tiles of a stage at the start of the next one; before the
    // first stage these are zero contributions: scale pair (0, 0) maps the
    // magic constant to exactly 0).  The next weight fragment is read one
    // fragment (four tiles) ahead; group 1's activation fragment b is read
    // right after its last use in group 0.
#pragma unroll
    for (int t = 0; t < 64; ++t) {
      const int gi = t >> 5, a = (t >> 2) & 7, b = t & 3, idx = t >> 2;
      dr[t & 3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[idx & 1], fx[b], cmagic, 0, 0, 0);
      if (b == 0 && idx < 15) rd_w(s, (idx + 1) >> 3, (idx + 1) & 7, fw[(idx + 1) & 1], swr[(idx + 1) & 3]);
      deq_tile((t + 62) & 63);
      if (gi == 0 && a == 7) {
        fx[b] = unpack_b64(*reinterpret_cast<const uint2*>(s + fx_off[1][b & 1] + (b >> 1) * 2048));
        const float ax = *reinterpret_cast<const float*>(s + xs_off + 1024 + 64 * b);
        xc[1][b] = make_float2(ax, -MAGIC_F * ax);
      }
    }
    // stage u + 1's codes landed before this stage began
    rd_first_codes(ring[(u + 1) % KT_NS]);
  }
  deq_tile(62);
  deq_tile(63);
  // drain the padding loads issued past the last stage before LDS is reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __syncthreads();
  kt_epilogue<OUT_F32, EPI>(acc, &ring[0][0], m0, n0, M, N, y, qa);
}

template <int ACT, int NT, int QM, int RT, int WB>
int launch_k1_instance(const void* x, const float* smooth_inv, const void* lora_down, int M, int K, int rank,
                       void* x_codes, void* x_scales, float* lora_act, size_t smem, int blocks, int waves,
                       hipStream_t st) {
  auto kern = k_quant_act_lora_down<ACT, NT, QM, RT, WB>;
  // Dynamic LDS above the default 64 KB needs an opt-in; it is made once per
  // instantiation for the whole 160 KB a CU offers (the size depends on K).
  static const bool attr_ok =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                          160 * 1024) == hipSuccess;
  if (!attr_ok && smem > 64 * 1024) return SVDQ_ERR_HIP;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(waves * 64), smem, st,
                     static_cast<const uint16_t*>(x), smooth_inv, static_cast<const uint16_t*>(lora_down), M, K,
                     rank, static_cast<uint8_t*>(x_codes), x_scales, lora_act);
  return SVDQ_OK;
}

template <int ACT, int NT, int QM, int RT>
int launch_k1_kernel(const void* x, const float* smooth_inv, const void* lora_down, int M, int K, int rank,
                     void* x_codes, void* x_scales, float* lora_act, size_t smem, hipStream_t st) {
  // Grids larger than the CU count run 8-wave blocks, two per CU, instead of
  // a second round of 16-wave blocks.
  const int rows = QM == Q_FP6 ? 32 * ((M + 31) / 32) : M;   // FP6: the padded last row block too
  const int blocks = (rows + K1_ROWS * RT - 1) / (K1_ROWS * RT);
  const int waves = (k1_waves<NT>() == 16 && blocks > svdq::device_cu_count()) ? 8 : k1_waves<NT>();
  // 32-row blocks of the 16-wave ranks launched as 8-wave blocks get the
  // 8-wave register budget (the 6-bit mode would spill in 128 VGPRs).
  if constexpr (RT == 2 && k1_waves<NT>() == 16) {
    if (waves == 8)
      return launch_k1_instance<ACT, NT, QM, RT, 8>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales,
                                                    lora_act, smem, blocks, waves, st);
  }
  return launch_k1_instance<ACT, NT, QM, RT, k1_waves<NT>()>(x, smooth_inv, lora_down, M, K, rank, x_codes,
                                                              x_scales, lora_act, smem, blocks, waves, st);
}

// Every block reads all of L1 (K x rank bf16), twice its own X bytes at rank
// 32, so once the 16-row blocks outnumber the CUs (M = 4608 and up) blocks of
// 32 rows, which use each L1 fragment for both row tiles, move a third fewer
// bytes per CU.  Up to rank 64 while the doubled reduction buffer fits LDS
// (with the GELU prologue too: its exp2-and-reciprocal form fits the same
// registers).
template <int ACT, int QM, int NT>
int launch_k1_nt(const void* x, const float* smooth_inv, const void* lora_down, int M, int K, int rank,
                  void* x_codes, void* x_scales, float* lora_act, hipStream_t st) {
  const size_t red1 = sizeof(float) * K1_MAX_WAVES * 2 * K1_ROWS * 16;
  const size_t smem1 = static_cast<size_t>(K) * sizeof(float) + red1;
  if constexpr (NT == 8) {
    // ranks 65..128 (8-wave blocks, 256 registers): 32-row blocks while they
    // still fill the chip read half the L1 bytes per row (at M = 16384 each
    // 16-row block would read 786 KB of L1 for 96 KB of X); 64-row blocks
    // would spill
    const size_t smem2 = static_cast<size_t>(K) * sizeof(float) + sizeof(float) * 8 * 2 * K1_ROWS * 2 * 16;
    if ((M + 2 * K1_ROWS - 1) / (2 * K1_ROWS) >= svdq::device_cu_count() && smem2 <= 160 * 1024)
      return launch_k1_kernel<ACT, NT, QM, 2>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act,
                                              smem2, st);
  }
  if constexpr (NT > 0 && NT <= 4) {
    bool many = (M + K1_ROWS - 1) / K1_ROWS > svdq::device_cu_count();
    // the 6-bit mode at ranks 49..64 fits its registers only as 8-wave
    // blocks, i.e. when the 32-row blocks themselves outnumber the CUs
    if (QM == Q_FP6 && NT == 4) many = (M + 2 * K1_ROWS - 1) / (2 * K1_ROWS) > svdq::device_cu_count();
    if (many && smem1 + red1 <= 160 * 1024)
      return launch_k1_kernel<ACT, NT, QM, 2>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act,
                                              smem1 + red1, st);
  }
  return launch_k1_kernel<ACT, NT, QM, 1>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act,
                                          smem1, st);
}

template <int ACT, int QM>
int launch_k1(const void* x, const float* smooth_inv, const void* lora_down, int M, int K, int rank,
              void* x_codes, void* x_scales, float* lora_act, hipStream_t st) {
  const size_t smem = static_cast<size_t>(K) * sizeof(float) + sizeof(float) * K1_MAX_WAVES * 2 * K1_ROWS * 16;
  if (smem > 160 * 1024) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  const int nt = rank / 16;
  int rc;
  if (nt == 0) rc = launch_k1_nt<ACT, QM, 0>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
  else if (nt <= 2) rc = launch_k1_nt<ACT, QM, 2>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
  else if (nt <= 4) rc = launch_k1_nt<ACT, QM, 4>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
  else if (nt <= 8) rc = launch_k1_nt<ACT, QM, 8>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
  else rc = launch_k1_nt<ACT, QM, 16>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
  if (rc != SVDQ_OK) return rc;
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

// ---------------------------------------------------------------------
// Unfused up projection (reference path for the fusion ablation):
// y = bf16(y + bf16(lora_act) lora_up^T), reading and rewriting the 16-bit
// output.  Block 128 x 128, 4 waves of 64 x 64, bf16 MFMA 32x32x16 computing
// the transposed tile (lora_up rows as the A operand) so a lane holds one
// output row and runs of four columns, loaded and stored as 8-byte chunks.
__global__ __launch_bounds__(256) void k_lora_up_add(const float* __restrict__ lora_act,
                                                     const uint16_t* __restrict__ lora_up, int M, int N,
                                                     int rank, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fr = lane & 31, fk = lane >> 5;
  const int nN = (N + 127) / 128;
  const int m0 = (blockIdx.x / nN) * 128 + (wave >> 1) * 64;
  const int n0 = (blockIdx.x % nN) * 128 + (wave & 1) * 64;
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = m0 + i * 32 + fr;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int c = n0 + j * 32 + 8 * bb + 4 * fk;
        uint2 v = make_uint2(0, 0);
        if (row < M && c < N) v = *reinterpret_cast<const uint2*>(y + static_cast<size_t>(row) * N + c);
        acc[i][j][4 * bb + 0] = bf16_bits_to_f32(v.x & 0xFFFFu);
        acc[i][j][4 * bb + 1] = bf16_bits_to_f32(v.x >> 16);
        acc[i][j][4 * bb + 2] = bf16_bits_to_f32(v.y & 0xFFFFu);
        acc[i][j][4 * bb + 3] = bf16_bits_to_f32(v.y >> 16);
      }
    }
  }
  for (int kk = 0; kk < rank; kk += 16) {
    const int kl = kk + fk * 8;
    v8bf la[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = m0 + i * 32 + fr;
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
    for (int j = 0; j < 2; ++j) {
      const int c = n0 + j * 32 + fr;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (c < N) u = *reinterpret_cast<const uint4*>(lora_up + static_cast<size_t>(c) * rank + kl);
      const v8bf ub = __builtin_bit_cast(v8bf, u);
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ub, la[i], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = m0 + i * 32 + fr;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int c = n0 + j * 32 + 8 * bb + 4 * fk;
        if (c >= N) continue;
        const uint32_t lo = bf16x2_bits(acc[i][j][4 * bb + 0], acc[i][j][4 * bb + 1]);
        const uint32_t hi = bf16x2_bits(acc[i][j][4 * bb + 2], acc[i][j][4 * bb + 3]);
        *reinterpret_cast<uint2*>(y + static_cast<size_t>(row) * N + c) = make_uint2(lo, hi);
      }
    }
  }
}

// LDS: the stage buffers, and in the epilogue the four 64 x 64 bf16 output
// tiles followed by the QKV epilogue's row sums (4 waves x 4 tiles x 16 rows).
constexpr size_t K2_SMEM_EPI = static_cast<size_t>(K2_WAVES) * K2_WM * K2_WN * 2 + K2_WAVES * K2_TB * 16 * 4;
constexpr size_t K2_SMEM = sizeof(K2Smem) > K2_SMEM_EPI ? sizeof(K2Smem) : K2_SMEM_EPI;

template <int OUT_F32, int NT, int EPI>
int launch_k2_t128(const void* xc, const void* xs, const void* wc, const void* ws, const float* la,
                    const void* lu, const void* bias, int M, int N, int K, int rank, void* y,
                    const QkvArgs& qa, hipStream_t st) {
  // the stage buffers exceed the default 64 KB of dynamic LDS: opt in once
  static const bool attr_ok = [] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k_gemm_w4a4_lora_up_t128<OUT_F32, NT, EPI>),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(K2_SMEM)) == hipSuccess;
  }();
  if (!attr_ok) return SVDQ_ERR_HIP;
  const int nb = ((N + K2_BN - 1) / K2_BN) * ((M + K2_BM - 1) / K2_BM);
  hipLaunchKernelGGL((k_gemm_w4a4_lora_up_t128<OUT_F32, NT, EPI>), dim3(nb), dim3(K2_THREADS), K2_SMEM, st,
                     static_cast<const uint8_t*>(xc), static_cast<const _Float16*>(xs),
                     static_cast<const uint8_t*>(wc), static_cast<const _Float16*>(ws), la,
                     static_cast<const uint16_t*>(lu), static_cast<const uint16_t*>(bias), M, N, K, rank, y, qa);
  return SVDQ_OK;
}

template <int OUT_F32, int NT, int EPI>
void launch_k2_t256(const void* xc, const void* xs, const void* wc, const void* ws, const float* la,
                    const void* lu, const void* bias, int M, int N, int K, int rank, void* y,
                    const QkvArgs& qa, hipStream_t st) {
  const int nb = ((N + KT_BN - 1) / KT_BN) * ((M + KT_BM - 1) / KT_BM);
  hipLaunchKernelGGL((k_gemm_w4a4_lora_up<OUT_F32, NT, EPI>), dim3(nb), dim3(KT_THREADS), 0, st,
                     static_cast<const uint8_t*>(xc), static_cast<const _Float16*>(xs),
                     static_cast<const uint8_t*>(wc), static_cast<const _Float16*>(ws), la,
                     static_cast<const uint16_t*>(lu), static_cast<const uint16_t*>(bias), M, N, K, rank, y, qa);
}

// 256 x 256 tiles when they occupy at least three quarters of the CUs and M
// is even (that form reads the activation scales as aligned pairs); 128 x 128
// tiles otherwise.  At 192 tiles of 256 x 256 (M = 4096, N = 3072) the two
// forms take the same time for K = 3072 and the large one is 4 % faster for
// K = 12288; far below that the small form's extra blocks win.
template <int OUT_F32, int EPI>
int launch_k2(const void* xc, const void* xs, const void* wc, const void* ws, const float* la,
              const void* lu, const void* bias, int M, int N, int K, int rank, void* y, const QkvArgs& qa,
              hipStream_t st) {
  const long nb256 = static_cast<long>((M + KT_BM - 1) / KT_BM) * ((N + KT_BN - 1) / KT_BN);
  const bool big = (M % 2 == 0) && nb256 >= 192;
  if (big) {
    if (rank == 0) launch_k2_t256<OUT_F32, 0, EPI>(xc, xs, wc, ws, la, lu, bias, M, N, K, rank, y, qa, st);
    else launch_k2_t256<OUT_F32, 1, EPI>(xc, xs, wc, ws, la, lu, bias, M, N, K, rank, y, qa, st);
  } else {
    const int rc = rank == 0
        ? launch_k2_t128<OUT_F32, 0, EPI>(xc, xs, wc, ws, la, lu, bias, M, N, K, rank, y, qa, st)
        : launch_k2_t128<OUT_F32, 1, EPI>(xc, xs, wc, ws, la, lu, bias, M, N, K, rank, y, qa, st);
    if (rc != SVDQ_OK) return rc;
  }
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

}  // namespace

namespace svdq {

int launch_quant_act_lora_down(const void* x, const float* smooth_inv, const void* lora_down, int M,
                               int K, int rank, int act, void* x_codes, void* x_scales,
                               float* lora_act, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (act == SVDQ_ACT_GELU_TANH)
    return launch_k1<SVDQ_ACT_GELU_TANH, Q_INT4>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
  return launch_k1<SVDQ_ACT_NONE, Q_INT4>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
}

int launch_quant_act_lora_down_mxfp4(const void* x, const float* smooth_inv, const void* lora_down, int M,
                                     int K, int rank, int act, void* x_codes, void* x_scales,
                                     float* lora_act, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (act == SVDQ_ACT_GELU_TANH)
    return launch_k1<SVDQ_ACT_GELU_TANH, Q_MXFP4>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
  return launch_k1<SVDQ_ACT_NONE, Q_MXFP4>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
}

int launch_quant_act_lora_down_fp6(const void* x, const float* smooth_inv, const void* lora_down, int M, int K,
                                   int rank, int act, void* x_fp6, void* x_scales, float* lora_act, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (act == SVDQ_ACT_GELU_TANH)
    return launch_k1<SVDQ_ACT_GELU_TANH, Q_FP6>(x, smooth_inv, lora_down, M, K, rank, x_fp6, x_scales, lora_act, st);
  return launch_k1<SVDQ_ACT_NONE, Q_FP6>(x, smooth_inv, lora_down, M, K, rank, x_fp6, x_scales, lora_act, st);
}

int launch_lora_down(const void* x, const float* smooth_inv, const void* lora_down, int M, int K, int rank,
                     int act, float* lora_act, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (act == SVDQ_ACT_GELU_TANH)
    return launch_k1<SVDQ_ACT_GELU_TANH, Q_NONE>(x, smooth_inv, lora_down, M, K, rank, nullptr, nullptr, lora_act, st);
  return launch_k1<SVDQ_ACT_NONE, Q_NONE>(x, smooth_inv, lora_down, M, K, rank, nullptr, nullptr, lora_act, st);
}

int launch_lora_up_add(const float* lora_act, const void* lora_up, int M, int N, int rank, void* y, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int nb = ((M + 127) / 128) * ((N + 127) / 128);
  hipLaunchKernelGGL(k_lora_up_add, dim3(nb), dim3(256), 0, st, lora_act, static_cast<const uint16_t*>(lora_up), M,
                     N, rank, static_cast<uint16_t*>(y));
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

int launch_gemm_w4a4_lora_up(const void* x_codes, const void* x_scales, const void* w_codes,
                             const void* w_scales, const float* lora_act, const void* lora_up,
                             const void* bias, int M, int N, int K, int rank, int out_dtype, void* y,
                             void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const QkvArgs qa{nullptr, nullptr, nullptr, nullptr, 0.f};
  if (out_dtype == SVDQ_OUT_F32)
    return launch_k2<1, 0>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, qa, st);
  return launch_k2<0, 0>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, qa, st);
}

int launch_gemm_w4a4_lora_up_qkv(const void* x_codes, const void* x_scales, const void* w_codes,
                                 const void* w_scales, const float* lora_act, const void* lora_up,
                                 const void* bias, const void* norm_q, const void* norm_k, const float* rope_cos,
                                 const float* rope_sin, float eps, int M, int N, int K, int rank, int out_dtype,
                                 void* y, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const QkvArgs qa{static_cast<const uint16_t*>(norm_q), static_cast<const uint16_t*>(norm_k), rope_cos, rope_sin,
                   eps};
  if (out_dtype == SVDQ_OUT_F32)
    return launch_k2<1, 1>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, qa, st);
  return launch_k2<0, 1>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, qa, st);
}

}  // namespace svdq
