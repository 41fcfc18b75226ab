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
//   Block tile BM (m) x 256 (n) with BM / 32 waves, each owning 64 x 128
//   outputs = 2 x 4 MFMA tiles of 32 x 32, computed transposed (weight rows
//   are the MFMA A operand, activation rows the B operand) so a lane ends
//   with one output row and runs of four output columns.  BM = 256 (8
//   waves, one block per CU) for large M; BM = 128 (4 waves, two blocks per
//   CU) when 256-row tiles would leave CUs idle.
//   The K loop runs in stages of 128 k (two MFMA k-steps of 64).  Operands
//   move from HBM straight into a ring of NS LDS stage buffers with LDS-DMA
//   buffer loads (no registers involved), NS - 1 stages ahead of the stage
//   being multiplied, so enough bytes are in flight to cover the memory
//   latency; a stage is released by one barrier per stage.
//
// Operand layout of the 32x32x64 FP4 MFMA (wave64): lane l supplies row
// l % 32 and the 32 k of block l / 32 (16 bytes, element j in nibble j, low
// nibble first) together with that (row, block)'s E8M0 scale in its scale
// register; C/D as for every 32x32 MFMA: lane l holds column l % 32, rows
// 8b + 4(l / 32) + i in register 4b + i.  An LDS-DMA load writes lane l's
// bytes at the wave's LDS base + size * l.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq.h"
#include "svdq_device.h"
#include "svdq_internal.h"

namespace {

constexpr int MX_BN = 256;                   // block tile columns (n)
constexpr int MX_WM = 64;                    // wave tile rows
constexpr int MX_WN = 128;                   // wave tile columns
constexpr int MX_TI = MX_WM / 32;            // 32x32 tiles per wave along m
constexpr int MX_TJ = MX_WN / 32;            // along n
constexpr int MX_KS = 128;                   // k per stage


// Per-stage LDS layout (bytes): activation codes [BM rows][64], weight codes
// [256 rows][64], activation scales [BM] dwords, weight scales [256] dwords,
// one dummy dword row [64] for padding scale loads.  Codes: 16-byte chunk
// c (= k 32c .. 32c + 31 of the stage, one MFMA block) of row r sits at
// chunk c ^ (((r >> 1) ^ (r >> 3)) & 3), which spreads fragment reads over
// all banks; the DMA loads apply that permutation on the global side.
template <int BM>
struct MxCfg {
  static constexpr int WAVES = BM / 32;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int NS = BM == 256 ? 4 : 3;                   // ring depth
  static constexpr int A_BYTES = BM * 64;
  static constexpr int B_BYTES = MX_BN * 64;
  static constexpr int SA_OFF = A_BYTES + B_BYTES;
  static constexpr int SB_OFF = SA_OFF + BM * 4;
  static constexpr int DUMMY_OFF = SB_OFF + MX_BN * 4;
  static constexpr int STAGE_BYTES = DUMMY_OFF + 256;
  static constexpr int A_INSTR = BM / 16 / WAVES;                // 1 KB code loads per wave
  static constexpr int B_INSTR = MX_BN / 16 / WAVES;
  static constexpr int S_TOTAL = BM / 64 + MX_BN / 64;           // 256-byte scale loads
  static constexpr int S_INSTR = (S_TOTAL + WAVES - 1) / WAVES;
  static constexpr int P = A_INSTR + B_INSTR + S_INSTR;          // DMA loads per wave per stage
  static constexpr size_t SMEM_MAIN = static_cast<size_t>(NS) * STAGE_BYTES;
  static constexpr size_t SMEM_EPI = static_cast<size_t>(WAVES) * MX_WM * MX_WN * 2;
  static_assert(SMEM_EPI <= SMEM_MAIN, "the output tiles reuse the stage ring");
};

__device__ __forceinline__ int mx_swz(int row, int chunk) { return chunk ^ (((row >> 1) ^ (row >> 3)) & 3); }

template <int OUT_F32, int HAS_RANK, int BM>
__global__ __launch_bounds__(MxCfg<BM>::THREADS, BM == 256 ? 1 : 2) void k_gemm_mxfp4_lora_up(
    const uint8_t* __restrict__ x_codes, const uint8_t* __restrict__ x_scales,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
    const float* __restrict__ lora_act, const uint16_t* __restrict__ lora_up,
    const uint16_t* __restrict__ bias, int M, int N, int K, int rank, void* __restrict__ y) {
  using C = MxCfg<BM>;
  // A statically sized ring (not dynamic LDS): with the slot as the first
  // index the compiler can prove that different slots do not overlap.
  __shared__ __align__(16) unsigned char ring[C::NS][C::STAGE_BYTES];
  unsigned char* const mx_smem_raw = &ring[0][0];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nM = (M + BM - 1) / BM, nN = (N + MX_BN - 1) / MX_BN;
  int tm, tn;
  xcd_tile(nM, nN, tm, tn);
  const int m0 = tm * BM, n0 = tn * MX_BN;
  const int S = K / MX_KS;
  const uint32_t Kb = static_cast<uint32_t>(K) / 2;     // code bytes per row
  const uint32_t Ks = static_cast<uint32_t>(K) / 32;    // scale bytes per row
  constexpr uint32_t OOB = 0x80000000u;

  const DmaRsrc a_rs = dma_rsrc(x_codes, static_cast<uint32_t>(static_cast<size_t>(M) * Kb));
  const DmaRsrc b_rs = dma_rsrc(w_codes, static_cast<uint32_t>(static_cast<size_t>(N) * Kb));
  const DmaRsrc sa_rs = dma_rsrc(x_scales, static_cast<uint32_t>(static_cast<size_t>(M) * Ks));
  const DmaRsrc sb_rs = dma_rsrc(w_scales, static_cast<uint32_t>(static_cast<size_t>(N) * Ks));

  // DMA roles.  Code load i of this wave covers 16 rows (1 KB): lane l
  // fetches row 16q + l / 4, chunk (l & 3) ^ swz(row), landing in slot l & 3.
  // Scale load j (of the stage's BM / 64 + 4) covers 64 rows of one operand.
  uint32_t a_off[C::A_INSTR], b_off[C::B_INSTR], s_off[C::S_INSTR];
#pragma unroll
  for (int i = 0; i < C::A_INSTR; ++i) {
    const int q = wave * C::A_INSTR + i;
    const int r = 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ (((r >> 1) ^ (r >> 3)) & 3);
    a_off[i] = (m0 + r < M) ? static_cast<uint32_t>(m0 + r) * Kb + 16u * c : OOB;
  }
#pragma unroll
  for (int i = 0; i < C::B_INSTR; ++i) {
    const int q = wave * C::B_INSTR + i;
    const int r = 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ (((r >> 1) ^ (r >> 3)) & 3);
    b_off[i] = (n0 + r < N) ? static_cast<uint32_t>(n0 + r) * Kb + 16u * c : OOB;
  }
  bool s_is_a[C::S_INSTR];
  int s_lds[C::S_INSTR];
#pragma unroll
  for (int i = 0; i < C::S_INSTR; ++i) {
    const int j = wave * C::S_INSTR + i;            // wave-uniform
    if (j < BM / 64) {
      const int r = 64 * j + lane;
      s_is_a[i] = true;
      s_off[i] = (m0 + r < M) ? static_cast<uint32_t>(m0 + r) * Ks : OOB;
      s_lds[i] = C::SA_OFF + 256 * j;
    } else if (j < C::S_TOTAL) {
      const int r = 64 * (j - BM / 64) + lane;
      s_is_a[i] = false;
      s_off[i] = (n0 + r < N) ? static_cast<uint32_t>(n0 + r) * Ks : OOB;
      s_lds[i] = C::SB_OFF + 256 * (j - BM / 64);
    } else {                                        // padding: keeps every wave's count equal
      s_is_a[i] = true;
      s_off[i] = OOB;
      s_lds[i] = C::DUMMY_OFF;
    }
  }

  // LDS byte addresses (wave-uniform) of this wave's DMA targets in slot 0.
  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[0][0]));
  uint32_t a_lds[C::A_INSTR], b_lds[C::B_INSTR], s_lds_a[C::S_INSTR];
#pragma unroll
  for (int i = 0; i < C::A_INSTR; ++i)
    a_lds[i] = __builtin_amdgcn_readfirstlane(ring0 + 1024 * (wave * C::A_INSTR + i));
#pragma unroll
  for (int i = 0; i < C::B_INSTR; ++i)
    b_lds[i] = __builtin_amdgcn_readfirstlane(ring0 + C::A_BYTES + 1024 * (wave * C::B_INSTR + i));
#pragma unroll
  for (int i = 0; i < C::S_INSTR; ++i) s_lds_a[i] = __builtin_amdgcn_readfirstlane(ring0 + s_lds[i]);

  // Issue the DMA loads of stage st into ring slot `slot` = st % NS (zeros
  // past K).
  auto issue_stage = [&](int st, int slot) {
    const uint32_t so_lds = static_cast<uint32_t>(slot) * C::STAGE_BYTES;
    const bool live = st < S;
    const uint32_t ko = static_cast<uint32_t>(st) * (MX_KS / 2);
    const uint32_t so = static_cast<uint32_t>(st) * (MX_KS / 32);
#pragma unroll
    for (int i = 0; i < C::A_INSTR; ++i)
      dma16(a_rs, a_lds[i] + so_lds, (live && a_off[i] != OOB) ? a_off[i] + ko : OOB);
#pragma unroll
    for (int i = 0; i < C::B_INSTR; ++i)
      dma16(b_rs, b_lds[i] + so_lds, (live && b_off[i] != OOB) ? b_off[i] + ko : OOB);
#pragma unroll
    for (int i = 0; i < C::S_INSTR; ++i)
      dma4(s_is_a[i] ? sa_rs : sb_rs, s_lds_a[i] + so_lds, (live && s_off[i] != OOB) ? s_off[i] + so : OOB);
  };

  v16f acc[MX_TI][MX_TJ];
  const int fr = lane & 31;      // fragment row within a 32-row tile
  const int fk = lane >> 5;      // which 32-k block of the k-step

  // The accumulators start as bias + bf16(lora_act) L2, computed while the
  // first stages load: a lane holds output row m0 + 64 wm + 32 i + fr and
  // columns 32 j + 8 bb + 4 fk + (0..3) of each 32-column tile.  The up
  // projection runs on bf16 MFMA 32x32x16 (K = rank in slices of 16),
  // transposed like the main product.  The bias and the first slice's
  // operands are requested before the stages' DMA, unconditionally at
  // clamped in-bounds addresses and masked afterwards (loads under per-lane
  // branches would each be waited for before the next is issued).
  const int mw = m0 + wm * MX_WM, nw = n0 + wn * MX_WN;
  uint2 bvr[MX_TJ][4];
  float4 lar[MX_TI][2];
  uint4 lur[MX_TJ];
  if (bias) {                                            // uniform; N % 8 == 0
#pragma unroll
    for (int j = 0; j < MX_TJ; ++j)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
        bvr[j][bb] = *reinterpret_cast<const uint2*>(bias + min(nw + j * 32 + 8 * bb + 4 * fk, N - 4));
  }
  auto rank_loads = [&](int kk) {                        // kk + 16 <= rank
    const int kl = kk + fk * 8;
#pragma unroll
    for (int i = 0; i < MX_TI; ++i) {
      const float4* p =
          reinterpret_cast<const float4*>(lora_act + static_cast<size_t>(min(mw + i * 32 + fr, M - 1)) * rank + kl);
      lar[i][0] = p[0];
      lar[i][1] = p[1];
    }
#pragma unroll
    for (int j = 0; j < MX_TJ; ++j)
      lur[j] = *reinterpret_cast<const uint4*>(lora_up + static_cast<size_t>(min(nw + j * 32 + fr, N - 1)) * rank + kl);
  };
  if constexpr (HAS_RANK) rank_loads(0);

#pragma unroll
  for (int st = 0; st < C::NS - 1; ++st) issue_stage(st, st);

#pragma unroll
  for (int i = 0; i < MX_TI; ++i)
#pragma unroll
    for (int j = 0; j < MX_TJ; ++j)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        float b4[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias && nw + j * 32 + 8 * bb + 4 * fk < N) {
          b4[0] = bf16_bits_to_f32(bvr[j][bb].x & 0xFFFFu);
          b4[1] = bf16_bits_to_f32(bvr[j][bb].x >> 16);
          b4[2] = bf16_bits_to_f32(bvr[j][bb].y & 0xFFFFu);
          b4[3] = bf16_bits_to_f32(bvr[j][bb].y >> 16);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][4 * bb + e] = b4[e];
      }
  if constexpr (HAS_RANK) {
    for (int kk = 0; kk < rank; kk += 16) {
      if (kk > 0) rank_loads(kk);
      v8bf la[MX_TI];
#pragma unroll
      for (int i = 0; i < MX_TI; ++i) {
        const bool ok = mw + i * 32 + fr < M;
        const float4 v0 = lar[i][0], v1 = lar[i][1];
        const float v[8] = {ok ? v0.x : 0.f, ok ? v0.y : 0.f, ok ? v0.z : 0.f, ok ? v0.w : 0.f,
                            ok ? v1.x : 0.f, ok ? v1.y : 0.f, ok ? v1.z : 0.f, ok ? v1.w : 0.f};
        la[i] = pack_bf16x8(v);
      }
#pragma unroll
      for (int j = 0; j < MX_TJ; ++j) {
        const uint4 u = nw + j * 32 + fr < N ? lur[j] : make_uint4(0, 0, 0, 0);
        const v8bf ub = __builtin_bit_cast(v8bf, u);
#pragma unroll
        for (int i = 0; i < MX_TI; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ub, la[i], acc[i][j], 0, 0, 0);
      }
    }
  }

  for (int st0 = 0; st0 < S; st0 += C::NS) {
#pragma unroll
    for (int u = 0; u < C::NS; ++u) {
      const int st = st0 + u;
      if (st >= S) break;
      // stage st has landed once at most (NS - 2) stages of this wave's
      // loads are outstanding; every wave waits for its own loads, then the
      // barrier makes all of them visible and frees slot (st - 1) % NS, which
      // this wave's finished reads of the previous stage no longer need.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(C::P * (C::NS - 2)));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue_stage(st + C::NS - 1, (u + C::NS - 1) % C::NS);

      const unsigned char* base = ring[u];
      const uint4* sa4 = reinterpret_cast<const uint4*>(base);
      const uint4* sb4 = reinterpret_cast<const uint4*>(base + C::A_BYTES);
      const uint32_t* sas = reinterpret_cast<const uint32_t*>(base + C::SA_OFF);
      const uint32_t* sbs = reinterpret_cast<const uint32_t*>(base + C::SB_OFF);
      uint32_t sxw[MX_TI], sww[MX_TJ];
#pragma unroll
      for (int i = 0; i < MX_TI; ++i) sxw[i] = sas[wm * MX_WM + i * 32 + fr];
#pragma unroll
      for (int j = 0; j < MX_TJ; ++j) sww[j] = sbs[wn * MX_WN + j * 32 + fr];
#pragma unroll
      for (int ks = 0; ks < MX_KS / 64; ++ks) {
        const int chunk = 2 * ks + fk;
        v8i xf[MX_TI], wf[MX_TJ];
#pragma unroll
        for (int i = 0; i < MX_TI; ++i) {
          const int r = wm * MX_WM + i * 32 + fr;
          const uint4 v = sa4[r * 4 + mx_swz(r, chunk)];
          xf[i] = v8i{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w),
                      0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < MX_TJ; ++j) {
          const int c = wn * MX_WN + j * 32 + fr;
          const uint4 v = sb4[c * 4 + mx_swz(c, chunk)];
          wf[j] = v8i{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w),
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
    }
  }
  // drain the padding loads issued past the last stage before LDS is reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __syncthreads();

  // ---- store.  A lane holds output row m and columns
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
          const int chunk = j * 4 + bb;                 // 16-byte chunk of the 256-byte tile row
          tile[rl * 32 + ((chunk ^ (rl & 15)) << 1) + fk] =
              make_uint2(bf16x2_bits(o[0], o[1]),
                         bf16x2_bits(o[2], o[3]));
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

template <int OUT_F32, int HAS_RANK, int BM>
int launch_mx_kernel(const void* x_codes, const void* x_scales, const void* w_codes, const void* w_scales,
                     const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K,
                     int rank, void* y, hipStream_t st) {
  using C = MxCfg<BM>;
  auto kern = k_gemm_mxfp4_lora_up<OUT_F32, HAS_RANK, BM>;
  const int nb = ((M + BM - 1) / BM) * ((N + MX_BN - 1) / MX_BN);
  hipLaunchKernelGGL(kern, dim3(nb), dim3(C::THREADS), 0, st, static_cast<const uint8_t*>(x_codes),
                     static_cast<const uint8_t*>(x_scales), static_cast<const uint8_t*>(w_codes),
                     static_cast<const uint8_t*>(w_scales), lora_act, static_cast<const uint16_t*>(lora_up),
                     static_cast<const uint16_t*>(bias), M, N, K, rank, y);
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

template <int OUT_F32, int HAS_RANK>
int launch_mx(const void* x_codes, const void* x_scales, const void* w_codes, const void* w_scales,
              const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K, int rank,
              void* y, hipStream_t st) {
  // 256-row tiles when they still give every CU at least one block
  const long nb256 = static_cast<long>((M + 255) / 256) * ((N + MX_BN - 1) / MX_BN);
  if (nb256 >= 256)
    return launch_mx_kernel<OUT_F32, HAS_RANK, 256>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias,
                                                     M, N, K, rank, y, st);
  return launch_mx_kernel<OUT_F32, HAS_RANK, 128>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias,
                                                   M, N, K, rank, y, st);
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
      return launch_mx<1, 1>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, st);
    return launch_mx<1, 0>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, st);
  }
  if (rank > 0)
    return launch_mx<0, 1>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, st);
  return launch_mx<0, 0>(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, rank, y, st);
}

}  // namespace svdq
