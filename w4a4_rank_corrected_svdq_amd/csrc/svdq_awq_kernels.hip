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
//   M <= 16 rows.  The inner sums run on bf16 MFMA 32x32x16: a nibble q
//   becomes the bf16 value 128 + q by OR-ing it into the bit pattern 0x4300
//   (128 = 1.0 x 2^7 has seven free mantissa bits), so four MFMAs per group
//   give D = sum (128 + q) x_hat exactly per product, and the kernel
//   subtracts (128 + z_g) X_g.  A block owns 32 output columns; its waves
//   split K in chunks of 8 groups and add their partial results in LDS in
//   wave order.  All loads of a chunk (16 contiguous code bytes per lane and
//   group) are issued before any is used, which keeps enough bytes in flight
//   to stream HBM.
//
// MFMA 32x32x16 bf16 layouts (wave64): A lane l holds row l % 32 and 8
// values of k chosen by l / 32; B lane l holds column l % 32 and the same k;
// D lane l holds column l % 32, rows 8 b + 4 (l / 32) + i in register
// 4 b + i.  Here rows are the input rows (M <= 16, the rest read as zero),
// columns the output channels, and lane half h = l / 32 takes k = 64 g +
// 32 h + 8 t + (0..7) in the t-th MFMA of group g (any permutation of k
// applied to both operands leaves the product unchanged).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq.h"
#include "svdq_device.h"
#include "svdq_internal.h"

namespace {

constexpr int AWQ_GROUP = 64;
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
    // the group's 64 inputs and scales arrive with 8 + 16 vector loads issued
    // together; the sum then runs in increasing k
    const uint4* xr = reinterpret_cast<const uint4*>(x + static_cast<size_t>(m) * K + g * AWQ_GROUP);
    const float4* sr = reinterpret_cast<const float4*>(inv_scale + g * AWQ_GROUP);
    uint4 xv[8];
    float4 sv[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = xr[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = sr[i];
    const uint32_t* xw = reinterpret_cast<const uint32_t*>(xv);
    const float* sf = reinterpret_cast<const float*>(sv);
    uint32_t hv[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t p = bf16x2_bits(bf16_bits_to_f32(xw[i] & 0xFFFFu) * sf[2 * i],
                                     bf16_bits_to_f32(xw[i] >> 16) * sf[2 * i + 1]);
      s += bf16_bits_to_f32(p & 0xFFFFu);
      s += bf16_bits_to_f32(p >> 16);
      hv[i] = p;
    }
    uint4* hr = reinterpret_cast<uint4*>(x_hat + static_cast<size_t>(m) * K + g * AWQ_GROUP);
#pragma unroll
    for (int i = 0; i < 8; ++i) hr[i] = make_uint4(hv[4 * i], hv[4 * i + 1], hv[4 * i + 2], hv[4 * i + 3]);
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

// Block = one tile of 32 output columns; its W waves split K in chunks of 8
// groups (wave w takes chunks w, w + W, ...).  Lane l = 32 h + c: column
// n0 + c; per group g it loads 16 bytes of codes (k in [64 g + 32 h, +32))
// and four 16-byte activation fragments (the same k, row c), then runs four
// 32x32x16 bf16 MFMAs (k offsets 8 t of each half), so both halves of every
// MFMA lie in group g.  D lane l holds column n0 + c and rows 8 b + 4 h + i.
template <bool VEC_SCALES>
__global__ __launch_bounds__(VEC_SCALES ? 1024 : 512) void k_awq_gemv(
    const uint16_t* __restrict__ x_hat, const float* __restrict__ xsum, const uint8_t* __restrict__ w_codes,
    const _Float16* __restrict__ w_scales, const uint8_t* __restrict__ w_zeros, const uint16_t* __restrict__ bias,
    int M, int N, int K, uint16_t* __restrict__ y) {
  __shared__ float part[16][64][8];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int n = blockIdx.x * 32 + c;                          // N % 32 == 0: always < N
  const int G = K / AWQ_GROUP;
  const int chunks = (G + 7) / 8;
  const uint32_t Kb = static_cast<uint32_t>(K) / 2;

  const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(w_codes), 0, static_cast<int>(static_cast<size_t>(N) * Kb), 0x00020000);
  // activation rows past M read as zero
  const __amdgpu_buffer_rsrc_t x_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x_hat), 0, static_cast<int>(static_cast<size_t>(M) * K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(w_scales), 0, static_cast<int>(static_cast<size_t>(N) * G * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t z_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(w_zeros), 0, static_cast<int>(static_cast<size_t>(N) * G), 0x00020000);
  const uint32_t w_row = static_cast<uint32_t>(n) * Kb + 16u * h;
  const uint32_t x_row = static_cast<uint32_t>(c) * K * 2 + 64u * h;   // A operand row = lane % 32

  v16f acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  for (int ch = wave; ch < chunks; ch += W) {
    const int g0 = ch * 8;
    // all loads of the chunk first; groups past G read as zeros and get scale 0
    uint4 wv[8];
    uint4 xa[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = g0 + j < G;
      wv[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            w_rs, ok ? w_row + 32u * (g0 + j) : 0x80000000u, 0, 0));
#pragma unroll
      for (int t = 0; t < 4; ++t)
        xa[j][t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 x_rs, ok ? x_row + 128u * (g0 + j) + 16u * t : 0x80000000u, 0, 0));
    }
    // scales (8 fp16) and zero points (8 bytes) of the chunk: one 16-byte and
    // one 8-byte load when rows start on 16-byte boundaries (G % 8 == 0),
    // else one load per group (past the row's end: unused values)
    const uint32_t so = static_cast<uint32_t>(n) * G + g0;
    _Float16 scl[8];
    uint8_t zpt[8];
    if constexpr (VEC_SCALES) {
      const uint4 sv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(s_rs, 2u * so, 0, 0));
      const uint2 zv = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(z_rs, so, 0, 0));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        scl[j] = reinterpret_cast<const _Float16*>(&sv)[j];
        zpt[j] = reinterpret_cast<const uint8_t*>(&zv)[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int g = min(g0 + j, G - 1);
      const uint32_t* wd = reinterpret_cast<const uint32_t*>(&wv[j]);
      v16f d;
#pragma unroll
      for (int v = 0; v < 16; ++v) d[v] = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, xa[j][t]), awq_nibbles_to_bf16(wd[t]), d,
                                                   0, 0, 0);
      if constexpr (!VEC_SCALES) {   // one load per group, at its use
        scl[j] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(s_rs, 2u * (so + j), 0, 0));
        zpt[j] = __builtin_amdgcn_raw_buffer_load_b8(z_rs, so + j, 0, 0);
      }
      const float s = (g0 + j < G) ? static_cast<float>(scl[j]) : 0.0f;
      const float cz = 128.0f + static_cast<float>(zpt[j]);
      const float4 x0 = *reinterpret_cast<const float4*>(xsum + g * AWQ_MAX_ROWS + 4 * h);
      const float4 x1 = *reinterpret_cast<const float4*>(xsum + g * AWQ_MAX_ROWS + 8 + 4 * h);
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * b + i] = fmaf(s, fmaf(-cz, xs[4 * b + i], d[4 * b + i]), acc[4 * b + i]);
    }
  }
  // rows 0..15 live in registers 0..7 (b = 0, 1); rows 16..31 are padding
#pragma unroll
  for (int v = 0; v < 8; ++v) part[wave][lane][v] = acc[v];
  __syncthreads();
  if (wave == 0) {
    const float bb = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      float t = part[0][lane][v];
      for (int w = 1; w < W; ++w) t += part[w][lane][v];
      const int m = 8 * (v >> 2) + 4 * h + (v & 3);
      if (m < M) y[static_cast<size_t>(m) * N + n] = static_cast<uint16_t>(f32_to_bf16_bits(t + bb));
    }
  }
}


// ---------------------------------------------------------------------
// Streaming form (K % 256 == 0).  A block owns 32 output columns and walks K
// in slots of 4 groups; each slot's bytes travel from HBM straight into a
// ring of AWD_NS LDS slots with LDS-DMA buffer loads (AWD_NS - 1 slots in
// flight), so a CU keeps tens of KB of weights in flight without holding
// them in registers: the 32 weight rows (128 bytes each), the 16 activation
// rows (512 bytes each; rows past M read as zero), the scales, zero points
// and row sums of the 4 groups.  Wave w computes group w of every slot
// (four 32x32x16 bf16 MFMAs, then the same dequantization as above) and the
// waves' partial results are added in LDS in wave order.
constexpr int AWD_NS = 4;
constexpr int AWD_W = 0;                       // slot layout (bytes): weights [32 rows][128]
constexpr int AWD_X = 4096;                    //   activations [16 rows][512]
constexpr int AWD_S = 12288;                   //   scales [32 rows][4] fp16
constexpr int AWD_Z = 12544;                   //   zero points [32 rows][4] u8 (+128 bytes of padding loads)
constexpr int AWD_XS = 12800;                  //   row sums [4 groups][16] fp32
constexpr int AWD_DUMMY = 13056;               //   target of the padding load
constexpr int AWD_SLOT = 13312;
constexpr int AWD_P = 4;                       // DMA loads per wave per slot
static_assert(AWD_NS * AWD_SLOT <= 160 * 1024 / 3, "three blocks per CU");

__global__ __launch_bounds__(256) void k_awq_gemv_stream(
    const uint16_t* __restrict__ x_hat, const float* __restrict__ xsum, const uint8_t* __restrict__ w_codes,
    const _Float16* __restrict__ w_scales, const uint8_t* __restrict__ w_zeros, const uint16_t* __restrict__ bias,
    int M, int N, int K, uint16_t* __restrict__ y) {
  __shared__ __align__(16) unsigned char ring[AWD_NS][AWD_SLOT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * 32;
  const int G = K / AWQ_GROUP;
  const int S = G / 4;
  const uint32_t Kb = static_cast<uint32_t>(K) / 2;
  constexpr uint32_t OOB = 0x80000000u;

  const DmaRsrc w_rs = dma_rsrc(w_codes, static_cast<uint32_t>(static_cast<size_t>(N) * Kb));
  const DmaRsrc x_rs = dma_rsrc(x_hat, static_cast<uint32_t>(static_cast<size_t>(M) * K * 2));
  // the small array this wave moves (wave-uniform choice, kept in scalar registers)
  const void* sm_base = wave == 0 ? static_cast<const void*>(w_scales)
                                  : wave == 1 ? static_cast<const void*>(w_zeros) : static_cast<const void*>(xsum);
  const uint32_t sm_bytes = static_cast<uint32_t>(wave == 0   ? static_cast<size_t>(N) * G * 2
                                                  : wave == 1 ? static_cast<size_t>(N) * G
                                                              : static_cast<size_t>(G) * AWQ_MAX_ROWS * 4);
  const DmaRsrc sm_rs = dma_rsrc(sm_base, sm_bytes);

  // DMA roles.  Weights: wave w moves rows 8w .. 8w + 7 (lane l: row
  // 8w + l / 8, landing at 16-byte position l % 8 of the row, which holds
  // chunk (l % 8) ^ (row % 8) of the slot's 128 bytes).  Activations: rows
  // 2w, 2w + 1 and 2w + 8, 2w + 9 (lane l: row + l / 32, position l % 32,
  // holding chunk (l % 32) ^ (row % 16)).  The XOR placements keep the
  // fragment reads below free of bank conflicts.  One 256-byte load per wave
  // for the small arrays: wave 0 the scales (lane l: row l / 2, 4 bytes),
  // wave 1 the zero points (lanes 0..31), wave 2 the row sums, wave 3 a
  // padding load of zeros, so that every wave issues AWD_P loads per slot.
  const int wr = 8 * wave + (lane >> 3);
  const uint32_t w_off0 = static_cast<uint32_t>(n0 + wr) * Kb + 16u * static_cast<uint32_t>((lane & 7) ^ (wr & 7));
  const int xra = 2 * wave + (lane >> 5), xrb = xra + 8;
  const uint32_t xq = 16u * static_cast<uint32_t>(lane & 31);
  const uint32_t xa_off0 = xra < M ? static_cast<uint32_t>(xra) * K * 2 + (xq ^ (16u * (xra & 15))) : OOB;
  const uint32_t xb_off0 = xrb < M ? static_cast<uint32_t>(xrb) * K * 2 + (xq ^ (16u * (xrb & 15))) : OOB;
  uint32_t sm_off0 = OOB, sm_step = 0;
  if (wave == 0) {
    sm_off0 = static_cast<uint32_t>(n0 + (lane >> 1)) * G * 2 + 4u * (lane & 1);
    sm_step = 8;
  } else if (wave == 1) {
    sm_off0 = lane < 32 ? static_cast<uint32_t>(n0 + lane) * G : OOB;
    sm_step = 4;
  } else if (wave == 2) {
    sm_off0 = 4u * lane;
    sm_step = 4 * AWQ_MAX_ROWS * 4;
  }
  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[0][0]));
  const uint32_t w_lds = __builtin_amdgcn_readfirstlane(ring0 + AWD_W + 1024 * wave);
  const uint32_t xa_lds = __builtin_amdgcn_readfirstlane(ring0 + AWD_X + 1024 * wave);
  const uint32_t xb_lds = __builtin_amdgcn_readfirstlane(ring0 + AWD_X + 4096 + 1024 * wave);
  const uint32_t sm_lds = __builtin_amdgcn_readfirstlane(
      ring0 + (wave == 0 ? AWD_S : wave == 1 ? AWD_Z : wave == 2 ? AWD_XS : AWD_DUMMY));
  auto issue = [&](int s, int slot) {
    const uint32_t so = static_cast<uint32_t>(slot) * AWD_SLOT;
    const bool live = s < S;
    dma16(w_rs, w_lds + so, live ? w_off0 + 128u * s : OOB);
    dma16(x_rs, xa_lds + so, (live && xa_off0 != OOB) ? xa_off0 + 512u * s : OOB);
    dma16(x_rs, xb_lds + so, (live && xb_off0 != OOB) ? xb_off0 + 512u * s : OOB);
    dma4(sm_rs, sm_lds + so, (live && sm_off0 != OOB) ? sm_off0 + sm_step * s : OOB);
  };

  v16f acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  const int j = wave;                            // group of the slot this wave computes
  const int wp = 16 * ((2 * j + h) ^ (c & 7));   // position of the lane's 16 code bytes in its weight row
  const int cr = c & 15;

#pragma unroll
  for (int s = 0; s < AWD_NS - 1; ++s) issue(s, s);
  int slot = 0;
  for (int s = 0; s < S; ++s) {
    // slot s has landed once at most NS - 2 slots of this wave's loads are
    // outstanding; the barrier publishes it and frees the slot of s - 1
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(AWD_P * (AWD_NS - 2)));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(s + AWD_NS - 1, slot == 0 ? AWD_NS - 1 : slot - 1);
    const unsigned char* base = ring[slot];
    const uint4 wq = *reinterpret_cast<const uint4*>(base + AWD_W + c * 128 + wp);
    uint4 xa[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int q = 8 * j + 4 * h + t;
      const uint4 v = *reinterpret_cast<const uint4*>(base + AWD_X + cr * 512 + 16 * (q ^ cr));
      xa[t] = c < 16 ? v : make_uint4(0u, 0u, 0u, 0u);   // A rows 16..31 are padding
    }
    const float sc = static_cast<float>(*reinterpret_cast<const _Float16*>(base + AWD_S + c * 8 + 2 * j));
    const float cz = 128.0f + static_cast<float>(base[AWD_Z + 4 * c + j]);
    const float4 x0 = *reinterpret_cast<const float4*>(base + AWD_XS + 64 * j + 16 * h);
    const float4 x1 = *reinterpret_cast<const float4*>(base + AWD_XS + 64 * j + 32 + 16 * h);
    const uint32_t* wd = reinterpret_cast<const uint32_t*>(&wq);
    v16f d0, d1;
#pragma unroll
    for (int v = 0; v < 16; ++v) { d0[v] = 0.f; d1[v] = 0.f; }
    // two independent chains of two MFMAs
    d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, xa[0]), awq_nibbles_to_bf16(wd[0]), d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, xa[1]), awq_nibbles_to_bf16(wd[1]), d1, 0, 0, 0);
    d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, xa[2]), awq_nibbles_to_bf16(wd[2]), d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, xa[3]), awq_nibbles_to_bf16(wd[3]), d1, 0, 0, 0);
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] = fmaf(sc, fmaf(-cz, xs[v], d0[v] + d1[v]), acc[v]);
    slot = slot == AWD_NS - 1 ? 0 : slot + 1;
  }
  // loads past the last slot land before the ring is reused for the sums
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __syncthreads();
  float (*part)[64][8] = reinterpret_cast<float (*)[64][8]>(&ring[0][0]);
#pragma unroll
  for (int v = 0; v < 8; ++v) part[wave][lane][v] = acc[v];
  __syncthreads();
  if (wave == 0) {
    const int n = n0 + c;
    const float bb = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const float t = ((part[0][lane][v] + part[1][lane][v]) + part[2][lane][v]) + part[3][lane][v];
      const int m = 8 * (v >> 2) + 4 * h + (v & 3);
      if (m < M) y[static_cast<size_t>(m) * N + n] = static_cast<uint16_t>(f32_to_bf16_bits(t + bb));
    }
  }
}

// ---------------------------------------------------------------------
// Single-row form (M = 1, K <= 8192: the one conditioning vector of the
// modulation layers).  Nothing is shared between output channels but x_hat,
// so each wave streams whole weight rows with the vector ALUs: lane l owns
// bytes 16 l of every 1 KB chunk c of a row, i.e. codes k0 = 2048 c + 32 l
// .. + 31, half of group g = 32 c + l / 2; its x_hat values stay in
// registers (packed bf16) for every row.  A wave takes awv_rows consecutive
// output channels with all their loads issued first.  Per lane and chunk
// d = sum (128 + q) x_hat over its 32 codes -- the MFMA form's offset codes,
// here as bf16 pairs in bf16 dot products into fp32 (four chains over the
// byte positions of its four code dwords, then added pairwise); the two
// lanes of a group add their d (lane ^ 1), t = d - (128 + z) X_g, and the
// even lanes sum s t over their chunks; a fixed tree over the even lanes and
// the bias give the output.
// Output channels per wave: six while a row is at most two 1 KB chunks
// (three waves per SIMD: at N = 18432 the 3072 waves are all resident in
// one round), two beyond (two waves per SIMD).
template <int CH> constexpr int awv_rows() { return CH <= 2 ? 6 : 2; }

// FUSED = 1 folds k_awq_act in: from x [K] and inv_scale [K] every block
// forms x_hat and the group sums X_g in LDS with the same arithmetic and
// order (x_hat = bf16(fp32(x * inv_scale)); X_g summed in fp32 in increasing
// k), so the output equals the two-kernel path's bit for bit.  Its x loads
// are issued first and the weight loads right behind them, so that forming
// x_hat waits only for the former, and the LDS barriers wait only for LDS.
template <int CH, int FUSED>                   // 1 KB chunks per weight row (K <= 2048 CH)
__global__ __launch_bounds__(256, CH <= 2 ? 3 : 2) void k_awq_gemv_row1(
    const uint16_t* __restrict__ xin, const float* __restrict__ xaux, const uint8_t* __restrict__ w_codes,
    const _Float16* __restrict__ w_scales, const uint8_t* __restrict__ w_zeros, const uint16_t* __restrict__ bias,
    int N, int K, uint16_t* __restrict__ y) {
  // xin: FUSED ? x : x_hat (one row, bf16); xaux: FUSED ? inv_scale [K] : xsum [K/64][16]
  __shared__ __align__(16) uint32_t xh_s[FUSED ? 1024 * CH : 4];   // x_hat pairs (k, k + 1)
  __shared__ float xg_s[FUSED ? 32 * CH : 1];        // X_g
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int gw = blockIdx.x * (blockDim.x >> 6) + (tid >> 6);
  constexpr int AWV_ROWS = awv_rows<CH>();
  const int n0 = AWV_ROWS * gw;
  const int Kb = K / 2;
  const int G = K / AWQ_GROUP;
  uint32_t xb[CH][16];                         // x_hat[k0 + 2 i] | x_hat[k0 + 2 i + 1] << 16
  float xs[CH];
  bool ok[CH];
  constexpr int XP = FUSED ? 4 * CH : 1;       // x pairs per thread: K / 2 <= 1024 CH over 256 threads
  uint32_t xr[XP];
  float2 ir[XP];
#pragma unroll
  for (int c = 0; c < CH; ++c) ok[c] = 1024 * c + 16 * lane < Kb;
  if constexpr (FUSED) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int pi = min(tid + 256 * i, Kb - 1);          // clamped; pairs past K / 2 are not stored
      xr[i] = reinterpret_cast<const uint32_t*>(xin)[pi];
      ir[i] = reinterpret_cast<const float2*>(xaux)[pi];
    }
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int k0 = 2048 * c + 32 * lane;
      uint4 v[4] = {};
      xs[c] = 0.f;
      if (ok[c]) {
        const uint4* p = reinterpret_cast<const uint4*>(xin + k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = p[i];
        xs[c] = xaux[(k0 / AWQ_GROUP) * AWQ_MAX_ROWS];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xb[c][4 * i] = v[i].x;
        xb[c][4 * i + 1] = v[i].y;
        xb[c][4 * i + 2] = v[i].z;
        xb[c][4 * i + 3] = v[i].w;
      }
    }
  }
  // Every load of the wave's rows is issued before any is used, at clamped
  // in-bounds addresses (rows past N read row N - 1, byte ranges past K the
  // row's first chunk), and masked afterwards: a load under a per-lane
  // branch would be waited for before the next one is issued.
  uint4 wq[AWV_ROWS][CH];
  uint16_t sr[AWV_ROWS][CH];
  uint8_t zr[AWV_ROWS][CH];
  uint16_t br[AWV_ROWS];
  // without a bias the loads read the scales (masked to +0 below), so that
  // no load sits under a branch
  const uint16_t* bsrc = bias ? bias : reinterpret_cast<const uint16_t*>(w_scales);
  const uint32_t bmask = bias ? 0xFFFFu : 0u;
#pragma unroll
  for (int j = 0; j < AWV_ROWS; ++j) {
    const size_t n = static_cast<size_t>(min(n0 + j, N - 1));
    br[j] = bsrc[n];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int gi = ok[c] ? 32 * c + (lane >> 1) : 0;
      const int bo = ok[c] ? 1024 * c + 16 * lane : 0;
      wq[j][c] = *reinterpret_cast<const uint4*>(w_codes + n * Kb + bo);
      sr[j][c] = reinterpret_cast<const uint16_t*>(w_scales)[n * G + gi];
      zr[j][c] = w_zeros[n * G + gi];
    }
  }
  if constexpr (FUSED) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int pi = tid + 256 * i;
      if (pi < Kb)
        xh_s[pi] = bf16x2_bits(bf16_bits_to_f32(xr[i] & 0xFFFFu) * ir[i].x, bf16_bits_to_f32(xr[i] >> 16) * ir[i].y);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (tid < G) {
      float sum = 0.f;
      for (int i = 0; i < AWQ_GROUP / 2; ++i) {
        const uint32_t pr = xh_s[(AWQ_GROUP / 2) * tid + i];
        sum += bf16_bits_to_f32(pr & 0xFFFFu);
        sum += bf16_bits_to_f32(pr >> 16);
      }
      xg_s[tid] = sum;
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int p0 = ok[c] ? 1024 * c + 16 * lane : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(&xh_s[p0 + 4 * i]);
        xb[c][4 * i] = v.x;
        xb[c][4 * i + 1] = v.y;
        xb[c][4 * i + 2] = v.z;
        xb[c][4 * i + 3] = v.w;
      }
      xs[c] = ok[c] ? xg_s[p0 / (AWQ_GROUP / 2)] : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < AWV_ROWS; ++j) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (!ok[c]) wq[j][c] = make_uint4(0, 0, 0, 0);
      const float scv = ok[c] ? static_cast<float>(__builtin_bit_cast(_Float16, sr[j][c])) : 0.f;
      const float zcv = static_cast<float>(zr[j][c]);
      const uint32_t w[4] = {wq[j][c].x, wq[j][c].y, wq[j][c].z, wq[j][c].w};
      // Byte b of a code dword holds codes 2 b (low nibble) and 2 b + 1; as
      // the bf16 pair (128 + q_2b, 128 + q_2b+1) -- 0x4300 | q is the bf16
      // value 128 + q -- it meets the packed x_hat pair of the same two k in
      // one bf16 dot product into fp32.  Four independent chains, one per
      // byte position, then (d0 + d1) + (d2 + d3).
      float dp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          // bytes (lo.b, 0, hi.b, 0), then 0x43 into bytes 1 and 3
          const uint32_t sel = 0x0C000C00u | (static_cast<uint32_t>(4 + b) << 16) | static_cast<uint32_t>(b);
          const uint32_t qp = __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
          dp[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, qp), __builtin_bit_cast(v2bf, xb[c][4 * i + b]),
                                                  dp[b], false);
        }
      }
      float d = (dp[0] + dp[1]) + (dp[2] + dp[3]);
      d += __shfl_xor(d, 1);
      // d = sum (128 + q) x_hat; t = d - (128 + z) X_g
      acc = fmaf(scv, fmaf(-(128.0f + zcv), xs[c], d), acc);
    }
    acc = (lane & 1) ? 0.f : acc;
#pragma unroll
    for (int o = 32; o >= 2; o >>= 1) acc += __shfl_xor(acc, o);
    const int n = n0 + j;
    if (lane == 0 && n < N) y[n] = static_cast<uint16_t>(f32_to_bf16_bits(acc + bf16_bits_to_f32(br[j] & bmask)));
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

int launch_awq_linear_row(const void* x, const float* inv_scale, const void* w_codes, const void* w_scales,
                          const void* w_zeros, const void* bias, int N, int K, void* y, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int ch = (K / 2 + 1023) / 1024;
  const int rows = ch <= 2 ? awv_rows<2>() : awv_rows<3>();
  const int blocks = (N + 4 * rows - 1) / (4 * rows);
  auto kern = ch == 1 ? k_awq_gemv_row1<1, 1> : ch == 2 ? k_awq_gemv_row1<2, 1> : ch == 3 ? k_awq_gemv_row1<3, 1>
                                                                                        : k_awq_gemv_row1<4, 1>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t*>(x), inv_scale,
                     static_cast<const uint8_t*>(w_codes), static_cast<const _Float16*>(w_scales),
                     static_cast<const uint8_t*>(w_zeros), static_cast<const uint16_t*>(bias), N, K,
                     static_cast<uint16_t*>(y));
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

int launch_awq_gemv(const void* x_hat, const float* xsum, const void* w_codes, const void* w_scales,
                    const void* w_zeros, const void* bias, int M, int N, int K, void* y, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (M == 1 && K <= 4 * 2048) {
    // one row: awv_rows output channels per wave, four waves per block
    const int ch = (K / 2 + 1023) / 1024;
    const int rows = ch <= 2 ? awv_rows<2>() : awv_rows<3>();
    const int blocks = (N + 4 * rows - 1) / (4 * rows);
    auto kern = ch == 1 ? k_awq_gemv_row1<1, 0> : ch == 2 ? k_awq_gemv_row1<2, 0> : ch == 3 ? k_awq_gemv_row1<3, 0>
                                                                                          : k_awq_gemv_row1<4, 0>;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t*>(x_hat), xsum,
                       static_cast<const uint8_t*>(w_codes), static_cast<const _Float16*>(w_scales),
                       static_cast<const uint8_t*>(w_zeros), static_cast<const uint16_t*>(bias), N, K,
                       static_cast<uint16_t*>(y));
    return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
  }
  if ((K / AWQ_GROUP) % 4 == 0) {
    hipLaunchKernelGGL(k_awq_gemv_stream, dim3(N / 32), dim3(256), 0, st, static_cast<const uint16_t*>(x_hat), xsum,
                       static_cast<const uint8_t*>(w_codes), static_cast<const _Float16*>(w_scales),
                       static_cast<const uint8_t*>(w_zeros), static_cast<const uint16_t*>(bias), M, N, K,
                       static_cast<uint16_t*>(y));
    return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
  }
  const int chunks = (K / AWQ_GROUP + 7) / 8;
  const bool vec = (K / AWQ_GROUP) % 8 == 0;
  const int max_waves = vec ? 16 : 8;                // the per-group scale loads need more registers
  const int waves = chunks < max_waves ? chunks : max_waves;
  auto kern = vec ? k_awq_gemv<true> : k_awq_gemv<false>;
  hipLaunchKernelGGL(kern, dim3(N / 32), dim3(waves * 64), 0, st, static_cast<const uint16_t*>(x_hat), xsum,
                     static_cast<const uint8_t*>(w_codes), static_cast<const _Float16*>(w_scales),
                     static_cast<const uint8_t*>(w_zeros), static_cast<const uint16_t*>(bias), M, N, K,
                     static_cast<uint16_t*>(y));
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

}  // namespace svdq
