// HIP kernels for the SVDQuant W4A4 linear on gfx950 (MI355X).
//
// Kernel 1 (k_quant_act_lora_down): smoothing, per-(token, group of 64)
//   symmetric INT4 quantization with nibble packing, and the rank-r down
//   projection X_hat L1 on bf16 MFMA, all from one read of each input element
//   (svdq-int4-flux.1-depth-dev model card, "Nunchaku Engine Design": the
//   quantizer and the down projection share their input).
// Kernel 2 (k_gemm_w4a4_lora_up): INT4 x INT4 GEMM on int8 MFMA with exact
//   int32 per-group products, per-group dequantization, and the up projection
//   (X_hat L1) L2 plus bias in the epilogue (same section: the up projection
//   and the 4-bit compute share their output).
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

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int GROUP = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return static_cast<uint32_t>(__builtin_bit_cast(unsigned short, b));
}

__device__ __forceinline__ v8bf pack_bf16x8(const float* v) {
  v8s s;
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = static_cast<short>(f32_to_bf16_bits(v[i]));
  return __builtin_bit_cast(v8bf, s);
}

__device__ __forceinline__ float gelu_tanh(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float u = k0 * (x + 0.044715f * x * x * x);
  return 0.5f * x * (1.0f + tanhf(u));
}

// =====================================================================
// Kernel 1
// =====================================================================
// Block: 16 token rows, 8 waves; wave w handles groups w, w+8, ... of K.
// Lane l works on row (l % 16) and the 16 consecutive k of its group at
// offset 16*(l/16); the four lanes of a row reduce the group absmax with two
// cross-lane exchanges.  The down projection treats the lane's 16 values as
// two 16x16x32 bf16 MFMA A-operands (k offsets 0..7 and 8..15 of its slice).
constexpr int K1_WAVES = 8;
constexpr int K1_ROWS = 16;

template <int ACT, int NT>
__global__ __launch_bounds__(K1_WAVES * 64) void k_quant_act_lora_down(
    const uint16_t* __restrict__ x, const float* __restrict__ smooth_inv,
    const uint16_t* __restrict__ lora_down, int M, int K, int rank,
    uint8_t* __restrict__ x_codes, _Float16* __restrict__ x_scales, float* __restrict__ lora_act) {
  __shared__ float red[K1_WAVES][2][16][16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * K1_ROWS;
  const int row = m0 + (lane & 15);
  const bool row_ok = row < M;
  const int kq = (lane >> 4) * 16;
  const int G = K / GROUP;
  const int ntiles = rank >> 4;

  v4f acc[NT > 0 ? NT : 1];
#pragma unroll
  for (int t = 0; t < (NT > 0 ? NT : 1); ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xrow = x + static_cast<size_t>(row_ok ? row : 0) * K;

  for (int g = wave; g < G; g += K1_WAVES) {
    const int k0 = g * GROUP + kq;
    uint4 raw0 = make_uint4(0, 0, 0, 0), raw1 = make_uint4(0, 0, 0, 0);
    if (row_ok) {
      raw0 = *reinterpret_cast<const uint4*>(xrow + k0);
      raw1 = *reinterpret_cast<const uint4*>(xrow + k0 + 8);
    }
    const float4* sp = reinterpret_cast<const float4*>(smooth_inv + k0);
    float4 s4[4] = {sp[0], sp[1], sp[2], sp[3]};
    const float* sv = reinterpret_cast<const float*>(s4);
    uint32_t w[8] = {raw0.x, raw0.y, raw0.z, raw0.w, raw1.x, raw1.y, raw1.z, raw1.w};
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
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float s32 = amax / 7.0f;
    const _Float16 sh = static_cast<_Float16>(s32);
    const float sf = static_cast<float>(sh);
    const float rcp = (sf == 0.f) ? 0.f : 1.0f / sf;
    uint32_t p0 = 0, p1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = fminf(fmaxf(rintf(xh[i] * rcp), -8.f), 7.f);
      const float q1 = fminf(fmaxf(rintf(xh[8 + i] * rcp), -8.f), 7.f);
      p0 |= (static_cast<uint32_t>(static_cast<int>(q0)) & 0xFu) << (4 * i);
      p1 |= (static_cast<uint32_t>(static_cast<int>(q1)) & 0xFu) << (4 * i);
    }
    if (row_ok) {
      *reinterpret_cast<uint2*>(x_codes + static_cast<size_t>(row) * (K / 2) + (k0 >> 1)) = make_uint2(p0, p1);
      if (lane < 16) x_scales[static_cast<size_t>(g) * M + row] = sh;
    }
    if constexpr (NT > 0) {
      const v8bf a0 = pack_bf16x8(xh);
      const v8bf a1 = pack_bf16x8(xh + 8);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < ntiles) {
          const uint16_t* bp = lora_down + static_cast<size_t>(t * 16 + (lane & 15)) * K + k0;
          const v8bf b0 = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(bp));
          const v8bf b1 = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(bp + 8));
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc[t], 0, 0, 0);
        }
      }
    }
  }

  if constexpr (NT > 0) {
    // Deterministic cross-wave reduction of the down projection, two rank
    // tiles (32 ranks) at a time, summed in wave order.
    for (int t0 = 0; t0 < ntiles; t0 += 2) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t == t0 + tt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][tt][4 * (lane >> 4) + i][lane & 15] = acc[t][i];
          }
        }
      }
      __syncthreads();
      const int tt = threadIdx.x >> 8;         // 0..1
      const int r = (threadIdx.x >> 4) & 15;   // row in tile
      const int c = threadIdx.x & 15;          // col in tile
      if (t0 + tt < ntiles && m0 + r < M) {
        float s = 0.f;
#pragma unroll
        for (int wv = 0; wv < K1_WAVES; ++wv) s += red[wv][tt][r][c];
        lora_act[static_cast<size_t>(m0 + r) * rank + (t0 + tt) * 16 + c] = s;
      }
      __syncthreads();
    }
  }
}

// =====================================================================
// Kernel 2
// =====================================================================
// Block tile 128 x 128, 4 waves in a 2 x 2 arrangement (64 x 64 per wave,
// 4 x 4 MFMA tiles of 16 x 16).  One group of 64 along K per step, double
// buffered in LDS: A = 128 rows x 32 packed bytes, B = 128 columns x 32
// packed bytes, plus the group's 128 + 128 fp16 scales.
//
// Unpacking: a packed dword holds 8 codes (byte j = code 2j low, 2j+1 high).
// (w << 4) & 0xF0F0F0F0 puts the even codes in the high nibble of each
// byte and w & 0xF0F0F0F0 the odd ones, so every int8 lane of the MFMA
// operand equals 16 * q with no sign extension; the product is 256 * P_g.
//
// Dequantization: the int8 MFMA's C operand is the constant 0x4B400000, the
// bit pattern of 1.5 * 2^23.  |256 * P_g| <= 2^20 < 2^22, so the int32 result
// read as fp32 is exactly 1.5 * 2^23 + 256 * P_g.  With a = s_w / 256 and
// b = -1.5 * 2^23 * a (both exact in fp32), fma(D, a, b) = s_w * P_g exactly
// (11 + 13 significant bits), and acc = fma(that, s_x, acc) adds the group.
constexpr int K2_BM = 128;
constexpr int K2_BN = 128;
constexpr int MAGIC_I = 0x4B400000;
constexpr float MAGIC_F = 12582912.0f;  // 1.5 * 2^23

__device__ __forceinline__ v4i unpack16(uint2 p) {
  v4i r;
  r[0] = static_cast<int>((p.x << 4) & 0xF0F0F0F0u);
  r[1] = static_cast<int>(p.x & 0xF0F0F0F0u);
  r[2] = static_cast<int>((p.y << 4) & 0xF0F0F0F0u);
  r[3] = static_cast<int>(p.y & 0xF0F0F0F0u);
  return r;
}

template <int OUT_F32, int NT>
__global__ __launch_bounds__(256) void k_gemm_w4a4_lora_up(
    const uint8_t* __restrict__ x_codes, const _Float16* __restrict__ x_scales,
    const uint8_t* __restrict__ w_codes, const _Float16* __restrict__ w_scales,
    const float* __restrict__ lora_act, const uint16_t* __restrict__ lora_up,
    const uint16_t* __restrict__ bias, int M, int N, int K, int rank, void* __restrict__ y) {
  __shared__ uint4 sA[2][K2_BM * 2];   // [row][2 x 16 B]
  __shared__ uint4 sB[2][K2_BN * 2];
  __shared__ _Float16 sSx[2][K2_BM];
  __shared__ _Float16 sSw[2][K2_BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * K2_BN;
  const int m0 = blockIdx.y * K2_BM;
  const int G = K / GROUP;
  const size_t Kb = static_cast<size_t>(K) / 2;

  // global -> LDS assignment: thread t moves 16 bytes of row t/2 for A and B
  const int lrow = tid >> 1, lhalf = tid & 1;
  const bool a_ok = (m0 + lrow) < M;
  const bool b_ok = (n0 + lrow) < N;
  const uint8_t* a_src = x_codes + static_cast<size_t>(a_ok ? m0 + lrow : 0) * Kb + lhalf * 16;
  const uint8_t* b_src = w_codes + static_cast<size_t>(b_ok ? n0 + lrow : 0) * Kb + lhalf * 16;

  auto load_stage = [&](int g, uint4& ra, uint4& rb, _Float16& rs) {
    ra = a_ok ? *reinterpret_cast<const uint4*>(a_src + static_cast<size_t>(g) * 32) : make_uint4(0, 0, 0, 0);
    rb = b_ok ? *reinterpret_cast<const uint4*>(b_src + static_cast<size_t>(g) * 32) : make_uint4(0, 0, 0, 0);
    if (tid < K2_BM) {
      rs = (m0 + tid < M) ? x_scales[static_cast<size_t>(g) * M + m0 + tid] : static_cast<_Float16>(0.f);
    } else {
      const int c = tid - K2_BM;
      rs = (n0 + c < N) ? w_scales[static_cast<size_t>(g) * N + n0 + c] : static_cast<_Float16>(0.f);
    }
  };
  auto store_stage = [&](int buf, const uint4& ra, const uint4& rb, const _Float16& rs) {
    sA[buf][tid] = ra;
    sB[buf][tid] = rb;
    if (tid < K2_BM) sSx[buf][tid] = rs;
    else sSw[buf][tid - K2_BM] = rs;
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const v4i cmagic = {MAGIC_I, MAGIC_I, MAGIC_I, MAGIC_I};

  {
    uint4 ra, rb;
    _Float16 rs;
    load_stage(0, ra, rb, rs);
    store_stage(0, ra, rb, rs);
  }
  __syncthreads();

  const int fr = lane & 15;      // fragment row / column within a 16-tile
  const int fk = lane >> 4;      // K slice (8 packed bytes) within the group
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    uint4 ra, rb;
    _Float16 rs;
    const bool more = (g + 1) < G;
    if (more) load_stage(g + 1, ra, rb, rs);

    const uint2* pA = reinterpret_cast<const uint2*>(&sA[buf][0]);
    const uint2* pB = reinterpret_cast<const uint2*>(&sB[buf][0]);
    v4i af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = unpack16(pA[(wm * 64 + i * 16 + fr) * 4 + fk]);
#pragma unroll
    for (int j = 0; j < 4; ++j) bfr[j] = unpack16(pB[(wn * 64 + j * 16 + fr) * 4 + fk]);
    float ca[4], cb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ca[j] = static_cast<float>(sSw[buf][wn * 64 + j * 16 + fr]) * (1.0f / 256.0f);
      cb[j] = -MAGIC_F * ca[j];
    }
    float sx[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) sx[i][r] = static_cast<float>(sSx[buf][wm * 64 + i * 16 + 4 * fk + r]);

#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bfr[j], cmagic, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float t = __builtin_fmaf(__int_as_float(d[r]), ca[j], cb[j]);
          acc[i][j][r] = __builtin_fmaf(t, sx[i][r], acc[i][j][r]);
        }
      }
    }

    if (more) store_stage(buf ^ 1, ra, rb, rs);
    __syncthreads();
  }

  // ---- epilogue: up projection (bf16 MFMA, K = rank in slices of 32) + bias
  if constexpr (NT > 0) {
    for (int kk = 0; kk < rank; kk += 32) {
      const int kl = kk + fk * 8;          // this lane's 8 k values
      const bool k_ok = kl < rank;         // rank % 32 == 16: upper half padded
      v8bf la[4], ub[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + wm * 64 + i * 16 + fr;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (k_ok && r < M) {
          const float4* p = reinterpret_cast<const float4*>(lora_act + static_cast<size_t>(r) * rank + kl);
          const float4 v0 = p[0], v1 = p[1];
          v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
          v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
        }
        la[i] = pack_bf16x8(v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = n0 + wn * 64 + j * 16 + fr;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (k_ok && c < N) u = *reinterpret_cast<const uint4*>(lora_up + static_cast<size_t>(c) * rank + kl);
        ub[j] = __builtin_bit_cast(v8bf, u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(la[i], ub[j], acc[i][j], 0, 0, 0);
    }
  }

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = n0 + wn * 64 + j * 16 + fr;
    if (c >= N) continue;
    const float bv = bias ? bf16_bits_to_f32(bias[c]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 64 + i * 16 + 4 * fk + r;
        if (row < M) {
          const float v = acc[i][j][r] + bv;
          if (OUT_F32) {
            reinterpret_cast<float*>(y)[static_cast<size_t>(row) * N + c] = v;
          } else {
            reinterpret_cast<uint16_t*>(y)[static_cast<size_t>(row) * N + c] =
                static_cast<uint16_t>(f32_to_bf16_bits(v));
          }
        }
      }
    }
  }
}

template <int ACT>
int launch_k1(const void* x, const float* smooth_inv, const void* lora_down, int M, int K, int rank,
              void* x_codes, void* x_scales, float* lora_act, hipStream_t st) {
  const dim3 grid((M + K1_ROWS - 1) / K1_ROWS), block(K1_WAVES * 64);
  const int nt = rank / 16;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, st, static_cast<const uint16_t*>(x), smooth_inv,
                       static_cast<const uint16_t*>(lora_down), M, K, rank,
                       static_cast<uint8_t*>(x_codes), static_cast<_Float16*>(x_scales), lora_act);
  };
  if (nt == 0) go(k_quant_act_lora_down<ACT, 0>);
  else if (nt <= 2) go(k_quant_act_lora_down<ACT, 2>);
  else if (nt <= 4) go(k_quant_act_lora_down<ACT, 4>);
  else if (nt <= 8) go(k_quant_act_lora_down<ACT, 8>);
  else go(k_quant_act_lora_down<ACT, 16>);
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

template <int OUT_F32>
int launch_k2(const void* xc, const void* xs, const void* wc, const void* ws, const float* la,
              const void* lu, const void* bias, int M, int N, int K, int rank, void* y, hipStream_t st) {
  const dim3 grid((N + K2_BN - 1) / K2_BN, (M + K2_BM - 1) / K2_BM), block(256);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, st, static_cast<const uint8_t*>(xc),
                       static_cast<const _Float16*>(xs), static_cast<const uint8_t*>(wc),
                       static_cast<const _Float16*>(ws), la, static_cast<const uint16_t*>(lu),
                       static_cast<const uint16_t*>(bias), M, N, K, rank, y);
  };
  if (rank == 0) go(k_gemm_w4a4_lora_up<OUT_F32, 0>);
  else go(k_gemm_w4a4_lora_up<OUT_F32, 1>);
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

}  // namespace

namespace svdq {

int launch_quant_act_lora_down(const void* x, const float* smooth_inv, const void* lora_down, int M,
                               int K, int rank, int act, void* x_codes, void* x_scales,
                               float* lora_act, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (act == SVDQ_ACT_GELU_TANH)
    return launch_k1<SVDQ_ACT_GELU_TANH>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
  return launch_k1<SVDQ_ACT_NONE>(x, smooth_inv, lora_down, M, K, rank, x_codes, x_scales, lora_act, st);
}

int launch_gemm_w4a4_lora_up(const void* x_codes, const void* x_scales, const void* w_codes,
                             const void* w_scales, const float* lora_act, const void* lora_up,
                             const void* bias, int M, int N, int K, int rank, int out_dtype, void* y,
                             void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (out_dtype == SVDQ_OUT_F32)
    return launch_k2<1>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, st);
  return launch_k2<0>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, st);
}

}  // namespace svdq
