// INT4 layer on the 6-bit MFMA, 256 x 192 output tiles, transposed form.
//
// The arithmetic is that of k_gemm_w4a4_fp6 (svdq_fp6_kernels.hip; the
// per-group integer product P_g of the layer's INT4 codes, "Nunchaku Engine
// Design", exact on the 6-bit MFMA, then fp32 dequantization, the up
// projection in the same accumulators, bias, one rounding).  What differs is
// the tiling, for layers with N = 3072 and the like: at M = 4096 their
// 256 x 256 tiles number 192, three quarters of the 256 CUs, while 256 x 192
// tiles number exactly 256.
//
// Transposed form: the weight fragment is the MFMA A operand and the
// activation fragment the B operand, so the 32 x 32 result holds channels
// down and tokens across: lane l holds token l % 32 and channels
// 8 b + 4 (l / 32) + i in register 4 b + i.  A lane's four registers of one
// b are four adjacent channels of one token -- one 8-byte store -- with the
// weights in the plain fragment layout (row block rb = channels
// 32 rb .. 32 rb + 31, the layout the activations use), so no panel order is
// needed for a 96-channel wave tile.
//
// Block: 256 tokens x 192 channels, 8 waves in a 4 (tokens) x 2 (channels)
// grid; a wave owns 64 tokens x 96 channels = 2 x 3 tiles of 32 x 32.
// Persistent grid and ring as in k_gemm_w4a4_fp6: stages of two groups of
// 64 k (or two 16-rank chunks), three LDS slots, LDS-DMA issued two stages
// ahead, seven loads per wave per stage:
//   group half:    the tile's 8 activation fragments (12 KB, runs 0..11, waves
//                  0-3) and 6 weight fragments (9 KB, runs 12..20, waves 4-6);
//                  wave 7's three runs are past every buffer (no bytes, the
//                  same load count);
//   low-rank half: lora_act [256 tokens][16 ranks] fp32 (runs 0..15) and
//                  lora_up [192 channels][16 ranks] bf16 (runs 16..21; runs 22,
//                  23 past the buffer);
//   auxiliary:     raw fp16 scales of the next stage (wave 0 activations,
//                  wave 1 weights: 256 per group, of which the tile uses 192),
//                  the tile's bias (waves 2-7).
// Dequantization per group: t = P_g s_w (exact: 13 x 11 significant bits),
// acc = fma(t, s_x, acc).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq.h"
#include "svdq_internal.h"

#include "svdq_device.h"

namespace {

constexpr int FRAG = 1536;
constexpr int T_BM = 256;                             // tokens per tile
constexpr int T_BN = 192;                             // channels per tile
constexpr int T_WAVES = 8;
constexpr int T_THREADS = T_WAVES * 64;
constexpr int T_GPS = 2;                              // groups (or 16-rank chunks) per stage
constexpr int T_NS = 3;                               // ring slots
constexpr int T_A = 8 * FRAG;                         // activation fragments of a group, then weights
constexpr int T_HALF = 24 * 1024;                     // a group's (or rank chunk's) area of a slot
constexpr int T_OPS = T_GPS * T_HALF;
constexpr int T_SC = T_OPS;                           // raw fp16 scales: x [2][256] | w [2][256]
constexpr int T_SLOT = T_SC + 2048;
constexpr int T_LA = 0;                               // lora_act [256][16] fp32 (64 B rows)
constexpr int T_LU = 16384;                           // lora_up [192][16] bf16 (32 B rows)
constexpr int T_CONV = T_GPS * 512;                   // fp32 scales of a stage: x [2][256] | w [2][256]
constexpr int T_DMA = 2 * 3 + 1;                      // loads per wave per stage
constexpr int T_STORES = 24;                          // buffer stores per lane at a tile's end
constexpr int T_MIN_STAGES = T_NS - 1;
constexpr int T_MAX_TILES = 256;
static_assert(T_A + 6 * FRAG <= 21 * 1024, "operand runs 0..20 hold a group's fragments");
static_assert(T_LU + T_BN * 32 <= 22 * 1024, "lora_up fills runs 16..21");
static_assert(T_DMA * (T_NS - 2) + T_STORES <= 63, "wait counts fit vmcnt");
static_assert(T_NS * T_SLOT + 2 * T_CONV * 4 + 2 * 256 * 2 + T_MAX_TILES * 4 <= 160 * 1024, "LDS of one CU");

__device__ __forceinline__ void dma16x3_t(const DmaRsrc& r, uint32_t lds_addr, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\ts_nop 4\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen offset:2048 lds"
      :: "s"(lds_addr), "v"(voff), "s"(r.w) : "memory", "m0");
}

// Tile of index t in the XCD-aware order (as k_gemm_w4a4_fp6's tile_of).
__device__ __forceinline__ void tile_of_t(int t, int nM, int nN, int& tm, int& tn) {
  const int nb = nM * nN;
  int u = t;
  if ((nb & 7) == 0) u = (t & 7) * (nb >> 3) + (t >> 3);
  constexpr int GM = 4;
  const int per = GM * nN;
  const int grp = u / per;
  const int first = grp * GM;
  const int gm = min(GM, nM - first);
  const int r = u - grp * per;
  tm = first + r % gm;
  tn = r / gm;
}

template <int OUT_F32>
__global__ __launch_bounds__(T_THREADS, 1) void k_gemm_w4a4_fp6_n192(
    const uint8_t* __restrict__ x_fp6, const _Float16* __restrict__ x_scales,
    const uint8_t* __restrict__ w_fp6, const _Float16* __restrict__ w_scales,
    const float* __restrict__ lora_act, const uint16_t* __restrict__ lora_up,
    const uint16_t* __restrict__ bias, int M, int N, int K, int rank, void* __restrict__ y) {
  __shared__ __align__(16) unsigned char ring[T_NS][T_SLOT];
  __shared__ __align__(16) float conv[2][T_CONV];
  __shared__ __align__(16) uint16_t bias_ring[2][256];    // bias of the tiles with even / odd index j
  __shared__ int tiles[T_MAX_TILES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int c = lane & 31, h = lane >> 5;
  const int nM = (M + T_BM - 1) / T_BM, nN = N / T_BN;
  const int ntiles = nM * nN;
  const int G = K / GROUP;
  const int NR = rank / 16;
  const int GS = (G + 1) / 2;
  const int SPT = max(GS + (NR + 1) / 2, T_MIN_STAGES);
  const int my_tiles = (ntiles - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                       static_cast<int>(gridDim.x);
  const int RBa = (M + 31) / 32;
  const int Mp = 32 * RBa;
  const int RBw = N / 32;
  constexpr uint32_t OOB = 0x80000000u;
  constexpr int ELEM = OUT_F32 ? 4 : 2;

  // operand role: waves 0-3 activations, 4-6 weights, 7 none (loads past the
  // end of the weight buffer)
  const bool opA = wave < 4;
  const DmaRsrc op_rs = dma_rsrc(opA ? static_cast<const void*>(x_fp6) : static_cast<const void*>(w_fp6),
                                 static_cast<uint32_t>(static_cast<size_t>(G) * (opA ? RBa : RBw) * FRAG));
  const DmaRsrc aux_rs =
      wave == 0 ? dma_rsrc(x_scales, static_cast<uint32_t>(static_cast<size_t>(G) * Mp * 2))
                : (wave == 1 ? dma_rsrc(w_scales, static_cast<uint32_t>(static_cast<size_t>(G) * N * 2))
                             : dma_rsrc(bias, bias ? static_cast<uint32_t>(N) * 2u : 0u));
  const DmaRsrc la_rs = dma_rsrc(lora_act, static_cast<uint32_t>(static_cast<size_t>(M) * rank * 4));
  const DmaRsrc lu_rs = dma_rsrc(lora_up, static_cast<uint32_t>(static_cast<size_t>(N) * rank * 2));
  const uint32_t y_bytes = static_cast<uint32_t>(static_cast<size_t>(M) * N * ELEM);
  const __amdgpu_buffer_rsrc_t y_rs = __builtin_amdgcn_make_buffer_rsrc(y, 0, static_cast<int>(y_bytes), 0x00020000);

  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[0][0]));
  const uint32_t bias0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&bias_ring[0][0]));

  for (int j = tid; j < my_tiles; j += T_THREADS) {
    int tm, tn;
    tile_of_t(static_cast<int>(blockIdx.x) + j * static_cast<int>(gridDim.x), nM, nN, tm, tn);
    tiles[j] = (tm << 16) | tn;
  }
  __syncthreads();
  auto tile_at = [&](int j) { return __builtin_amdgcn_readfirstlane(tiles[j < my_tiles ? j : 0]); };

  const uint32_t op_run0 = 1024u * static_cast<uint32_t>(opA ? 3 * wave : 3 * wave - 12);
  const uint32_t op_gstride = static_cast<uint32_t>(opA ? RBa : RBw) * FRAG;
  const uint32_t op_lds = __builtin_amdgcn_readfirstlane(ring0 + 1024 * 3 * wave);
  const uint32_t aux_lds = __builtin_amdgcn_readfirstlane(ring0 + T_SC + 1024 * wave);   // waves 0-1
  const uint32_t bias_lds = __builtin_amdgcn_readfirstlane(bias0 + 256u * (wave & 1));   // waves 2-7
  const uint32_t aux_lim = wave == 0 ? 2u * Mp : 2u * N;
  auto fresh_lane = [&]() {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  auto scale_off = [&](int t, int g) {
    const uint32_t b0 = wave == 0 ? 2u * T_BM * static_cast<uint32_t>(t >> 16)
                                  : 2u * T_BN * static_cast<uint32_t>(t & 0xFFFF);
    return static_cast<uint32_t>(g) * aux_lim + b0;
  };
  auto bias_off = [&](int t) {
    return bias != nullptr ? 2u * T_BN * static_cast<uint32_t>(t & 0xFFFF) + 256u * (wave & 1) : OOB;
  };
  auto scale_load = [&](uint32_t lds, int t, int g0) {
    const int ln = fresh_lane();
    const int g = g0 + (ln >> 5);
    const uint32_t v = g0 >= 0 && g < G ? scale_off(t, g) + 16u * (ln & 31) : OOB;
    dma16(aux_rs, lds, v);
  };

  int ji = 0, li = 0;
  uint32_t so = 0;
  int ti = tile_at(0), tnx = tile_at(1);
  // first operand run of tile t; wave 7 has none
  auto op_base_of = [&](int t) {
    if (wave == 7) return OOB;
    return (opA ? 8u * FRAG * static_cast<uint32_t>(t >> 16) : 6u * FRAG * static_cast<uint32_t>(t & 0xFFFF)) +
           op_run0;
  };
  uint32_t op_cur = op_base_of(ti);
  uint32_t aux_cur = wave < 2 ? scale_off(ti, 2) : bias_off(ti);
  const uint32_t aux_step = wave < 2 ? 2u * aux_lim : 0u;
  const uint32_t op_step = wave == 7 ? 0u : 2u * op_gstride;
  auto advance = [&]() {
    so = so == (T_NS - 1) * T_SLOT ? 0u : so + T_SLOT;
    if (++li == SPT) {
      li = 0;
      ++ji;
      ti = tnx;
      tnx = tile_at(ji + 1);
      op_cur = op_base_of(ti);
      aux_cur = wave < 2 ? scale_off(ti, 2) : bias_off(ti);
    } else {
      op_cur += op_step;
      aux_cur += aux_step;
    }
  };
  auto issue = [&]() {
    const bool live = ji < my_tiles;
    const uint32_t blds = __builtin_amdgcn_readfirstlane(bias_lds + 512u * static_cast<uint32_t>(ji & 1));
    if (live && 2 * (li + 2) <= G) {
      const int ln = fresh_lane();
      dma16x3_t(op_rs, __builtin_amdgcn_readfirstlane(op_lds + so), op_cur + 16u * ln);
      dma16x3_t(op_rs, __builtin_amdgcn_readfirstlane(op_lds + so + T_HALF),
                (wave == 7 ? OOB : op_cur + op_gstride) + 16u * ln);
      if (wave < 2)
        dma16(aux_rs, __builtin_amdgcn_readfirstlane(aux_lds + so),
              aux_cur + static_cast<uint32_t>(ln >> 5) * aux_lim + 16u * (ln & 31));
      else
        dma4(aux_rs, blds, aux_cur + 4u * ln);
      advance();
      return;
    }
    const int ln = fresh_lane();
    const uint32_t l16 = 16u * ln;
    const int tmi = ti >> 16, tni = ti & 0xFFFF;
    if (li < GS || !live) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int g = 2 * li + hh;
        const uint32_t base = __builtin_amdgcn_readfirstlane(
            live && g < G && wave != 7 ? op_base_of(ti) + static_cast<uint32_t>(g) * op_gstride : OOB);
        dma16x3_t(op_rs, __builtin_amdgcn_readfirstlane(op_lds + so + T_HALF * hh), base + l16);
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ch = 2 * (li - GS) + hh;                     // rank chunk; >= NR: padding
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const int q = 3 * wave + i;
          const bool isla = q < 16;
          const bool real = isla || q < 16 + T_BN / 32;
          const int row0 = isla ? T_BM * tmi + 16 * q : T_BN * tni + 32 * (q - 16);
          const uint32_t base = __builtin_amdgcn_readfirstlane(
              ch < NR && real ? (static_cast<uint32_t>(row0) * rank + 16u * ch) * (isla ? 4u : 2u) : OOB);
          const uint32_t lds = __builtin_amdgcn_readfirstlane(op_lds + 1024 * i + so + T_HALF * hh);
          if (isla)
            dma16(la_rs, lds, base + static_cast<uint32_t>(ln >> 2) * static_cast<uint32_t>(rank * 4) + 16u * (ln & 3));
          else
            dma16(lu_rs, lds, base + static_cast<uint32_t>(ln >> 1) * static_cast<uint32_t>(rank * 2) + 16u * (ln & 1));
        }
      }
    }
    if (wave < 2) {
      const int lnext = li + 1;
      const bool same = live && lnext < GS, nxt = live && lnext == SPT && ji + 1 < my_tiles;
      scale_load(__builtin_amdgcn_readfirstlane(aux_lds + so), same ? ti : tnx, same ? 2 * lnext : (nxt ? 0 : -1));
    } else {
      dma4(aux_rs, blds, (live ? bias_off(ti) : OOB) + 4u * ln);
    }
    advance();
  };
  auto convert_scales = [&](int slot, int buf) {
    int t = tid;
    asm volatile("" : "+v"(t));
    const _Float16* raw = reinterpret_cast<const _Float16*>(&ring[slot][T_SC]);
    const float lo = static_cast<float>(raw[t]), hi = static_cast<float>(raw[t + T_THREADS]);
    conv[buf][t] = lo;
    conv[buf][t + T_THREADS] = hi;
  };

  // acc[ct][a]: channel tile ct (of the wave's 3), token tile a (of 2)
  v16f acc[3][2];
#pragma unroll
  for (int ct = 0; ct < 3; ++ct)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ct][a][e] = 0.f;

  const uint32_t x_off = (2 * wm) * FRAG + 16u * lane;         // activation fragments (B operand)
  const uint32_t w_off = T_A + (3 * wn) * FRAG + 16u * lane;   // weight fragments (A operand)
  const v16f zero = {};

  if (wave < 2) scale_load(__builtin_amdgcn_readfirstlane(aux_lds + (T_NS - 1) * T_SLOT), ti, 0);
#pragma unroll
  for (int k = 0; k < T_NS - 1; ++k) issue();
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(T_DMA * (T_NS - 2)));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  convert_scales(T_NS - 1, 0);

  int s = 0, sc = 0, since_end = 8;
  auto stage_top = [&]() {
    if (since_end < T_NS - 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(T_DMA * (T_NS - 2) + T_STORES));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(T_DMA * (T_NS - 2)));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue();
    convert_scales(sc, (s + 1) & 1);
  };
  // The same in two parts, so that a group stage reads its first
  // fragments between them: their LDS latency then overlaps the DMA issue and
  // the scale conversion (the DMA's inline assembly keeps every LDS access in
  // program order around it).
  auto stage_wait = [&]() {
    if (since_end < T_NS - 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(T_DMA * (T_NS - 2) + T_STORES));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(T_DMA * (T_NS - 2)));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto stage_issue = [&]() {
    issue();
    convert_scales(sc, (s + 1) & 1);
  };
  auto stage_end = [&]() {
    ++s;
    sc = sc == T_NS - 1 ? 0 : sc + 1;
    ++since_end;
  };

  for (int j = 0; j < my_tiles; ++j) {
    const int tt = __builtin_amdgcn_readfirstlane(tiles[j]);
    const int mw = T_BM * (tt >> 16) + 64 * wm, cw = T_BN * (tt & 0xFFFF) + 96 * wn;   // wave-uniform

    // ---- the tile's groups ----
    for (int l = 0; l < GS; ++l, stage_end()) {
      stage_wait();
      // The stage's 12 tiles (two groups x 6) in one sequence u: group u / 6,
      // then (channel tile 0, token tile 0), (0, 1), (1, 0), ...  A weight
      // fragment serves two consecutive tiles and is read one tile pair
      // ahead; the MFMA of tile u + 1 is issued before tile u is dequantized.
      // A tile's channel scales are read four at a time (one per b) when its
      // channel tile starts; a lane's token scales once per group.
      const unsigned char* sl = ring[sc];
      const float* cv = conv[s & 1];
      auto rd_frag = [&](uint32_t off) {
        const uint4 lo = *reinterpret_cast<const uint4*>(sl + off);
        const uint2 hi = *reinterpret_cast<const uint2*>(sl + off + 1024 - 8 * lane);
        return v8i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                   static_cast<int>(hi.x), static_cast<int>(hi.y), 0, 0};
      };
      v8i xfr[2];
      xfr[0] = rd_frag(x_off);
      xfr[1] = rd_frag(x_off + FRAG);
      v8i wfr[3];
      wfr[0] = rd_frag(w_off);
      stage_issue();
      v16f dr[2];
      float swv[4][4];
      float sxv[2];
#pragma unroll
      for (int u = 0; u < 13; ++u) {
        if (u < 12) {
          const int hg = u / 6, ct = (u % 6) >> 1, a = u & 1;
          if (a == 0 && ct < 2) wfr[ct + 1] = rd_frag(T_HALF * hg + w_off + (ct + 1) * FRAG);
          // cbsz = blgp = 3: both operands E3M2; E8M0 scales 127 (= 1)
          dr[u & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wfr[ct], xfr[a], zero, 3, 3, 0, 127, 0, 127);
          if (u == 5) {
            xfr[0] = rd_frag(T_HALF + x_off);
            xfr[1] = rd_frag(T_HALF + x_off + FRAG);
            wfr[0] = rd_frag(T_HALF + w_off);
          }
        }
        if (u > 0) {
          const int v = u - 1, hv = v / 6, ct = (v % 6) >> 1, a = v & 1;
          if (v % 6 == 0) {
            sxv[0] = cv[T_BM * hv + 64 * wm + c];
            sxv[1] = cv[T_BM * hv + 64 * wm + 32 + c];
          }
          if (a == 0) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const float4 w4 =
                  *reinterpret_cast<const float4*>(cv + T_GPS * T_BM + 256 * hv + 96 * wn + 32 * ct + 8 * b + 4 * h);
              swv[b][0] = w4.x; swv[b][1] = w4.y; swv[b][2] = w4.z; swv[b][3] = w4.w;
            }
          }
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int e = 4 * b + i;
              acc[ct][a][e] = __builtin_fmaf(dr[v & 1][e] * swv[b][i], sxv[a], acc[ct][a][e]);
            }
        }
      }
    }

    // ---- the up projection, two 16-rank chunks per stage; padding stages ----
    for (int l = GS; l < SPT; ++l, stage_end()) {
      stage_top();
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        if (2 * (l - GS) + hh >= NR) break;
        const unsigned char* sl = ring[sc] + T_HALF * hh;
        // A = lora_up rows (channels n_w + 32 ct + l % 32, ranks 8 h .. 8 h + 7
        // of the chunk), B = bf16(lora_act) rows (tokens m_w + 32 a + l % 32)
        const int ln = fresh_lane();
        const int lc = ln & 31, lh = ln >> 5;
        v8bf la[2], lu[3];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const float4* p = reinterpret_cast<const float4*>(sl + T_LA + (64 * wm + 32 * a + lc) * 64 + 32 * lh);
          const float4 v0 = p[0], v1 = p[1];
          const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          la[a] = pack_bf16x8(v);
        }
#pragma unroll
        for (int ct = 0; ct < 3; ++ct)
          lu[ct] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(sl + T_LU + (96 * wn + 32 * ct + lc) * 32 + 16 * lh));
        v16f dr[2];
#pragma unroll
        for (int u = 0; u < 7; ++u) {
          if (u < 6) dr[u & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lu[u >> 1], la[u & 1], zero, 0, 0, 0);
          if (u > 0) {
            const int v = u - 1;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[v >> 1][v & 1][e] += dr[v & 1][e];
          }
        }
      }
    }

    // ---- end of the tile: bias, rounding, store ----
    {
      // The lane holds token mw + 32 a + l % 32 and channels cw + 32 ct +
      // 8 b + 4 h .. + 3; tokens past M fall past the end of y.  The bias
      // ring entry of tile j is rewritten only by the stages of tile j + 2.
      const int ln = fresh_lane();
      const int lc = ln & 31, lh = ln >> 5;
      const uint32_t vbase = mw + lc < M
                                 ? ((static_cast<uint32_t>(mw) + static_cast<uint32_t>(lc)) * static_cast<uint32_t>(N) +
                                    static_cast<uint32_t>(cw) + 4u * lh) * ELEM
                                 : OOB;
#pragma unroll
      for (int ct = 0; ct < 3; ++ct)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint2 bu = *reinterpret_cast<const uint2*>(&bias_ring[j & 1][96 * wn + 32 * ct + 8 * b + 4 * lh]);
          const float bv[4] = {bf16_bits_to_f32(bu.x & 0xFFFFu), bf16_bits_to_f32(bu.x >> 16),
                               bf16_bits_to_f32(bu.y & 0xFFFFu), bf16_bits_to_f32(bu.y >> 16)};
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const uint32_t off =
                vbase + (static_cast<uint32_t>(32 * a) * static_cast<uint32_t>(N) + 32u * ct + 8u * b) * ELEM;
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = acc[ct][a][4 * b + i] + bv[i];
            if (OUT_F32) {
              const v4f ov = v4f{o[0], o[1], o[2], o[3]};
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, ov), y_rs, off, 0, 0);
            } else {
              typedef int v2i_ __attribute__((ext_vector_type(2)));
              const v2i_ ov = v2i_{static_cast<int>(bf16x2_bits(o[0], o[1])), static_cast<int>(bf16x2_bits(o[2], o[3]))};
              __builtin_amdgcn_raw_buffer_store_b64(ov, y_rs, off, 0, 0);
            }
          }
        }
#pragma unroll
      for (int ct = 0; ct < 3; ++ct)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[ct][a][e] = 0.f;
      since_end = 0;
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
}

}  // namespace

namespace svdq {

int launch_gemm_w4a4_fp6_n192(const void* x_fp6, const void* x_scales, const void* w_fp6, const void* w_scales,
                              const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K,
                              int rank, int out_dtype, void* y, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int tiles = ((M + T_BM - 1) / T_BM) * (N / T_BN);
  const int cus = device_cu_count() & ~7;
  const int grid = tiles < cus ? tiles : (cus > 0 ? cus : tiles);
  if ((tiles + grid - 1) / grid > T_MAX_TILES) return SVDQ_ERR_UNSUPPORTED_SHAPE;
#define SVDQ_K2T(OF)                                                                                          \
  hipLaunchKernelGGL((k_gemm_w4a4_fp6_n192<OF>), dim3(grid), dim3(T_THREADS), 0, st,                          \
                     static_cast<const uint8_t*>(x_fp6), static_cast<const _Float16*>(x_scales),              \
                     static_cast<const uint8_t*>(w_fp6), static_cast<const _Float16*>(w_scales), lora_act,    \
                     static_cast<const uint16_t*>(lora_up), static_cast<const uint16_t*>(bias), M, N, K, rank, y)
  if (out_dtype == SVDQ_OUT_F32) SVDQ_K2T(1);
  else SVDQ_K2T(0);
#undef SVDQ_K2T
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

int fp6_n192_preferred(int M, int N) {
  // 256 x 192 tiles when N allows them and they fill the CUs in fewer
  // rounds: the time is the number of rounds times a tile's time, and a
  // 256 x 192 tile takes 0.875 of a 256 x 256 tile's (measured on MI355X
  // over 3 and 4 full rounds at 16384 x 3072 -> 3072: the per-stage barrier,
  // DMA issue and waits do not shrink with the tile's 3/4 of the work)
  if (N <= 0 || N % T_BN != 0 || M <= 0) return 0;
  const int cus = device_cu_count();
  const long long nM = (M + 255) / 256;
  const long long r256 = (nM * ((N + 255) / 256) + cus - 1) / cus;
  const long long r192 = (nM * (N / T_BN) + cus - 1) / cus;
  return 0.875 * static_cast<double>(r192) < static_cast<double>(r256) ? 1 : 0;
}

int fp6_route(int M, int N) {
  // Below half a round of 256 x 256 tiles the int8 engine's 128 x 128 form
  // (two blocks per CU) keeps more CUs busy than either 6-bit form: measured
  // on MI355X at M = 256-2048, N = 3072 (K = 512-12288) it takes 0.67-0.87 of
  // the 6-bit time, while at 192 or more tiles of 256 x 256 (M = 1024 and
  // 2048 at N = 12288) the 6-bit engine is faster (0.77-0.81 of int8's).
  if (M <= 0 || N <= 0) return 0;
  const long long tiles256 = static_cast<long long>((M + 255) / 256) * ((N + 255) / 256);
  if (2 * tiles256 < device_cu_count()) return 2;
  return fp6_n192_preferred(M, N);
}

}  // namespace svdq
