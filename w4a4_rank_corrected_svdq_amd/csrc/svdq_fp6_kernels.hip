// INT4 layer on gfx950's 6-bit float matrix cores.
//
// The W4A4 product of the layer (svdq-int4-flux.1-depth-dev model card,
// "Nunchaku Engine Design": 4-bit compute fused with the up projection) is a
// sum of products of integer codes in [-8, 7].  Every such integer is a
// value of the 6-bit float format E3M2 (sign, 3 exponent bits with bias 3,
// 2 mantissa bits: 1 = 1.0 x 2^0, 5 = 1.25 x 2^2, 7 = 1.75 x 2^2,
// 8 = 1.0 x 2^3), and gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 multiplies
// E3M2 operands exactly and accumulates their 64 products in fp32, where an
// integer sum of magnitude <= 4096 is exact.  So the per-group integer
// product P_g comes out of one 6-bit MFMA per 32 x 32 tile, bit for bit the
// integer result, at the 6-bit rate (about 1.75 times the int8 rate per
// 64-k group measured on MI355X).  The codes are the layer's INT4 codes; only
// their container changes, from a nibble to a 6-bit field.
//
// Operand container ("fragment layout"), for a [rows][K] code matrix:
//   buffer [K/64][RB][1536 bytes], one 1536-byte fragment per (group g,
//   row block rb of 32 rows).  Lane l = r + 32 h of a fragment holds row r of
//   the block and the 32 codes of k = 64 g + 32 h + j, j = 0..31, packed as
//   a 192-bit little-endian string with code j at bits 6j .. 6j + 5 --
//   exactly the MFMA operand of lane l.  Its dwords 0..3 sit at byte 16 l of
//   the fragment and dwords 4..5 at byte 1024 + 8 l, so that a wave reads a
//   fragment with one 16-byte and one 8-byte LDS read per lane, both
//   conflict-free.
//   Activations: row block rb holds rows 32 rb .. 32 rb + 31 (RB =
//   ceil(M / 32); rows past M hold +0).  Weights: rows are grouped in panels
//   of 128 output channels, and row block 4 p + t holds channels
//   128 p + 4 r + t (r = 0..31), so that in kernel 2 a lane's four output
//   columns of a wave tile are adjacent (RB = 4 ceil(N / 128); channels past
//   N hold +0).
//
// Kernel 1 is k_quant_act_lora_down in its FP6 mode (svdq_kernels.hip): the
//   nibble kernel's smoothing, quantizer, scales and down projection, with
//   the codes written in the fragment layout.
// Kernel 2 (k_gemm_w4a4_fp6, below): P_g on the 6-bit MFMA, per-group
//   dequantization in fp32, bias and up projection in the same accumulators.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "svdq.h"
#include "svdq_internal.h"

#include "svdq_device.h"

namespace {

constexpr int FRAG = 1536;

// 32x32 MFMA layouts (wave64) used below:
//   A operand: lane l holds row l % 32 and the k slice l / 32 (32 codes for
//              the 6-bit MFMA with K = 64, 8 values for the bf16 MFMA with
//              K = 16);
//   B operand: lane l holds column l % 32 and the same k slice;
//   C/D:       lane l holds column l % 32, rows 8 b + 4 (l / 32) + i in
//              register 4 b + i (b, i = 0..3).
// Checked on the device with random integer operands against a host sum.

// =====================================================================
// Kernel 2
// =====================================================================
// Output tile 256 (m) x 256 (n), 8 waves in a 4 (m) x 2 (n) grid, one block
// per CU (two waves per SIMD); each wave owns 64 x 128 outputs = 2 x 4
// tiles of 32 x 32.  The activation fragment is the MFMA A operand and the
// weight fragment the B operand, so a lane holds one output column per tile
// and 16 rows; with the weights' panel order the four tiles of a wave give a
// lane the four adjacent columns n_w + 4 (l % 32) .. + 3.
//
// One group of 64 k is one 6-bit MFMA per tile (C = 0), giving P_g exactly
// in fp32.  Dequantization: t = P_g s_x (exact: 13 x 11 significant bits)
// and acc = fma(t, s_w, acc), one rounding per group -- the same two fp32
// operations per output and group as the int8 kernel, without its
// magic-constant conversion.
//
// Persistent grid: one block per CU walks the output tiles t = blockIdx.x,
// blockIdx.x + gridDim.x, ... as one continuous sequence of stages.  A stage
// carries two groups of 64 k (the second may be past K when K / 64 is odd),
// or two 16-rank chunks of the low-rank branch; a tile's stages are its
// ceil(G / 2) group stages, then ceil(rank / 32) low-rank stages (at least
// two stages per tile; empty ones pad).  Every stage moves 48 KB from HBM
// into a ring of F_NS LDS slots by LDS-DMA buffer loads, issued F_NS - 1
// stages ahead, seven per wave:
//   group half h:    the tile's 8 activation and 8 weight fragments of
//                    group 2 j + h (contiguous 12 KB runs in the fragment
//                    layout), three 1 KB runs per wave;
//   low-rank half h: lora_act [256 rows][16 ranks] fp32 and lora_up
//                    [256 columns][16 ranks] bf16 of chunk 2 j + h, added
//                    into the same accumulators on bf16 MFMA;
// plus one auxiliary load: wave 0 the raw fp16 activation scales and wave 1
// the weight scales of the stage after the issued one (1 KB each: a lane
// half per group), waves 2-7 the issued stage's tile's bias into a ring of
// two per-tile entries (every stage of a tile reloads the same bytes).  So
// at the top of stage s only stage s's loads must have landed; the barrier
// publishes them and the fp32 scales converted during stage s - 1, and
// frees the slot of stage s - 1 for stage s + 2.
// After a tile's last stage the wave adds the bias, rounds, and stores its
// 64 x 128 outputs with buffer stores (32 per lane; rows past M and columns
// past N fall outside the buffer and are dropped), then starts the next
// tile, whose first stages are already loading: the store overlaps them.
// Stores count in the same vmcnt as the loads, so the wait at a stage adds
// 32 to its count when a tile ended within the last F_NS - 1 stages (at
// most one can, with F_NS - 1 or more stages per tile).
constexpr int F_BM = 256;
constexpr int F_BN = 256;
constexpr int F_WAVES = 8;
constexpr int F_THREADS = F_WAVES * 64;
constexpr int F_GPS = 2;                              // groups (or 16-rank chunks) per stage
constexpr int F_NS = 3;                               // ring slots, one stage each
constexpr int F_A = 8 * FRAG;                         // 12288: activation fragments of a group
constexpr int F_HALF = 24 * 1024;                     // operand bytes of one group (or rank chunk)
constexpr int F_OPS = F_GPS * F_HALF;                 // operand bytes of a stage
constexpr int F_SC = F_OPS;                           // raw fp16 scales of the next stage: x [2][256] | w [2][256]
constexpr int F_SLOT = F_SC + 2048;
constexpr int F_LA = 0;                               // low-rank half: lora_act [256][16] fp32 (64 B rows)
constexpr int F_LU = 16384;                           //                lora_up [256][16] bf16 (32 B rows)
constexpr int F_CONV = F_GPS * (F_BM + F_BN);         // fp32 scales of a stage: x [2][256] | w [2][256]
constexpr int F_DMA = 2 * 3 + 1;                      // loads per wave per stage
constexpr int F_STORES = 32;                          // buffer stores per lane at a tile's end
constexpr int F_MIN_STAGES = F_NS - 1;
constexpr int F_MAX_TILES = 256;                      // tiles per block (the host checks)
static_assert(F_HALF / 1024 == 3 * F_WAVES, "three 1 KB operand loads per wave per group");
static_assert(F_LU + 256 * 32 == F_HALF, "a low-rank chunk fills a group's operand area");
static_assert(F_SLOT % 16 == 0, "slots stay 16-byte aligned");
static_assert(F_DMA * (F_NS - 2) + F_STORES <= 63, "wait counts fit vmcnt");
static_assert(F_NS * F_SLOT + 2 * F_CONV * 4 + 2 * F_BN * 2 + F_MAX_TILES * 4 <= 160 * 1024, "LDS of one CU");

// Three consecutive 1 KB LDS-DMA runs (16 bytes per lane each) under one M0
// write: the instruction offsets 0, 1024, 2048 advance the buffer offset and
// the LDS address alike, and the buffer range check sees voff + offset, so a
// voff past the end drops all three.
__device__ __forceinline__ void dma16x3(const DmaRsrc& r, uint32_t lds_addr, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\ts_nop 4\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen offset:2048 lds"
      :: "s"(lds_addr), "v"(voff), "s"(r.w) : "memory", "m0");
}

// Output tile of tile index t: the XCD-aware order of xcd_tile, applied to t
// (the block that runs tile t sits on XCD t % 8, as t = blockIdx.x + j *
// gridDim.x with gridDim.x a multiple of 8).
__device__ __forceinline__ void tile_of(int t, int nM, int nN, int& tm, int& tn) {
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

// The MLP chain's epilogue (EPI = 1): instead of storing Y, the block
// turns its output tile into the next layer's kernel-1 outputs -- bf16(Y),
// tanh-GELU, the next layer's smoothing and per-(row, group of 64) INT4
// quantizer, codes in the 6-bit containers -- and the tile's 256-column
// slice of the next layer's down projection, a partial that a second kernel
// sums over the column slices in order.  The next layer's K is this layer's N.
struct ChainArgs {
  const float* smooth_inv;   // [N] the next layer's 1 / lambda
  const uint16_t* lora_down; // [rank][N] bf16, the next layer's L1^T
  int rank;                  // the next layer's rank
  uint8_t* x_fp6;            // [N/64][ceil(M/32)][1536] codes of the next layer's input
  _Float16* x_scales;        // [N/64][32 ceil(M/32)]
  float* partials;           // [ceil(N/256)][M][rank]
};
constexpr int C_TS = 2 * F_BN + 16;                   // staging row stride in bytes (bank spread)

// The fused QKV epilogue (EPI = 2; "Bringing Nunchaku 4-bit Diffusion
// Inference to Diffusers", "Quantizing models with structural rewrites": one
// operator takes the QKV projection, the Q / K normalization and the rotary
// embedding together).  The output columns
// are Q heads, then K heads, then V heads of 128 columns (N = 3 heads 128);
// a wave's 128 columns are one head.  After bias, each Q or K row is scaled
// by 1 / sqrt(mean of its 128 squares + eps) and the head's bf16 norm
// weights, then adjacent column pairs (2 j, 2 j + 1) are rotated by
// cos / sin[row][j] when the tables are given; V is stored as projected.
struct QkvArgs6 {
  const uint16_t* gq;        // [128] bf16 norm weights of the Q heads
  const uint16_t* gk;        // [128] bf16 norm weights of the K heads
  const float* cos;          // [M][64] fp32 or NULL (no rotation)
  const float* sin;          // [M][64] fp32
  float eps;
};
constexpr int Q_HEAD = 128;
constexpr int Q_TAB = F_BM * 256;                     // bytes of one staged rotary table (256 rows x 64 fp32)
static_assert(2 * Q_TAB <= F_NS * F_SLOT, "both rotary tables fit the idle ring");

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// Sum over the 32 lanes of each wave half, the same value in all of them:
// quad swaps (lane ^ 1, ^ 2), then the mirrors within 8 and within 16 lanes
// (each pairs a lane with one in the other half of its 8 or 16), then lane
// ^ 16 by swizzle (bit-mask mode: and 0x1F, xor 0x10).
__device__ __forceinline__ float sum32(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  return v;
}
static_assert((F_BM + 32) * C_TS <= F_NS * F_SLOT,
              "the chain's staging tile and a 32-rank L1 slice fit the idle ring");

// EPI: 0 store Y, 1 the MLP chain's epilogue, 2 the fused QKV epilogue.
template <int OUT_F32, int EPI>
__global__ __launch_bounds__(F_THREADS, 1) void k_gemm_w4a4_fp6(
    const uint8_t* __restrict__ x_fp6, const _Float16* __restrict__ x_scales,
    const uint8_t* __restrict__ w_fp6, const _Float16* __restrict__ w_scales,
    const float* __restrict__ lora_act, const uint16_t* __restrict__ lora_up,
    const uint16_t* __restrict__ bias, int M, int N, int K, int rank, void* __restrict__ y, ChainArgs ca,
    QkvArgs6 qa) {
  __shared__ __align__(16) unsigned char ring[F_NS][F_SLOT];
  __shared__ __align__(16) float conv[2][F_CONV];
  __shared__ __align__(16) uint16_t bias_ring[2][F_BN];   // bias of the tiles with even / odd index j
  __shared__ int tiles[F_MAX_TILES];                      // this block's tiles: tm << 16 | tn

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int c = lane & 31, h = lane >> 5;
  const int nM = (M + F_BM - 1) / F_BM, nN = (N + F_BN - 1) / F_BN;
  const int ntiles = nM * nN;
  const int G = K / GROUP;
  const int NR = rank / 16;
  const int GS = (G + 1) / 2;                                 // group stages per tile
  const int SPT = max(GS + (NR + 1) / 2, F_MIN_STAGES);      // stages per tile
  const int my_tiles = (ntiles - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                       static_cast<int>(gridDim.x);
  const int RBa = (M + 31) / 32;
  const int Mp = 32 * RBa;
  const int RBb = 4 * ((N + 127) / 128);
  constexpr uint32_t OOB = 0x80000000u;
  constexpr int ELEM = OUT_F32 ? 4 : 2;

  // Buffer resources: each wave moves one operand in group stages
  // (activations for waves 0-3, weights for 4-7) and one auxiliary array
  // (activation scales for wave 0, weight scales for wave 1, bias for 2-7).
  const bool opA = wave < 4;
  const DmaRsrc op_rs = dma_rsrc(opA ? static_cast<const void*>(x_fp6) : static_cast<const void*>(w_fp6),
                                 static_cast<uint32_t>(static_cast<size_t>(G) * (opA ? RBa : RBb) * FRAG));
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

  // The block's tiles, t = blockIdx.x + j gridDim.x, in LDS (read at tile
  // changes, not recomputed in the loop).
  for (int j = tid; j < my_tiles; j += F_THREADS) {
    int tm, tn;
    tile_of(static_cast<int>(blockIdx.x) + j * static_cast<int>(gridDim.x), nM, nN, tm, tn);
    tiles[j] = (tm << 16) | tn;
  }
  __syncthreads();
  auto tile_at = [&](int j) { return __builtin_amdgcn_readfirstlane(tiles[j < my_tiles ? j : 0]); };

  // DMA roles (wave-uniform).  In a group half waves 0-3 move the 12 KB of
  // activation fragments and waves 4-7 the 12 KB of weight fragments, three
  // 1 KB runs each (run r of the operand: bytes 1024 r .. + 1023 of its
  // contiguous 12 KB); in a low-rank half runs 0..15 of the 24 are lora_act
  // (16 rows of 64 bytes each) and 16..23 lora_up (32 rows of 32 bytes).
  // The auxiliary load: wave 0 the activation scales and wave 1 the weight
  // scales of the two groups of the stage after the issued one (lane half
  // hl = lane / 32 takes the second group's 512 bytes), waves 2-7 a 256-byte
  // half of the issued tile's bias (waves 4-7 repeat 2-3).
  const uint32_t op_run0 = 1024u * static_cast<uint32_t>(opA ? 3 * wave : 3 * wave - 12);
  const uint32_t op_gstride = static_cast<uint32_t>(opA ? RBa : RBb) * FRAG;
  const uint32_t op_lds = __builtin_amdgcn_readfirstlane(ring0 + 1024 * 3 * wave);
  const uint32_t aux_lds = __builtin_amdgcn_readfirstlane(ring0 + F_SC + 1024 * wave);   // waves 0-1
  const uint32_t bias_lds = __builtin_amdgcn_readfirstlane(bias0 + 256u * (wave & 1));   // waves 2-7
  const uint32_t aux_lim = wave == 0 ? 2u * Mp : 2u * N;         // bytes per group of a scale array
  // The lane index, recomputed where it is used outside the group section
  // (an empty asm hides that it is loop-invariant), so that the compiler
  // does not keep every per-lane offset of the DMA, low-rank and store
  // paths in registers across the loop.
  auto fresh_lane = [&]() {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  const uint32_t lane16 = 16u * lane;
  // scale-array byte offset of group g of tile t (waves 0-1)
  auto scale_off = [&](int t, int g) {
    const uint32_t b0 = wave == 0 ? 2u * F_BM * static_cast<uint32_t>(t >> 16)
                                  : 2u * F_BN * static_cast<uint32_t>(t & 0xFFFF);
    return static_cast<uint32_t>(g) * aux_lim + b0;
  };
  auto bias_off = [&](int t) {
    return bias != nullptr ? 2u * F_BN * static_cast<uint32_t>(t & 0xFFFF) + 256u * (wave & 1) : OOB;
  };
  // the auxiliary load of waves 0-1: groups g0, g0 + 1 (lane halves);
  // groups past G, or g0 < 0, read as zeros
  auto scale_load = [&](uint32_t lds, int t, int g0) {
    const int ln = fresh_lane();
    const int g = g0 + (ln >> 5);
    const uint32_t v = g0 >= 0 && g < G ? scale_off(t, g) + 16u * (ln & 31) : OOB;
    dma16(aux_rs, lds, v);
  };

  // Issue cursor: the stage being issued is stage li of tile ji (tile
  // coordinates ti; those of the following tile tnx), at slot byte offset
  // so.  In the common case -- the issued stage and the one after it are
  // full group stages of a live tile -- the operand runs start at op_cur
  // and the scale load at aux_cur, both advanced by two groups per stage;
  // every other stage takes the general path, which also re-bases both at
  // a tile change.
  int ji = 0, li = 0;
  uint32_t so = 0;
  int ti = tile_at(0), tnx = tile_at(1);
  auto op_base_of = [&](int t) {
    return 8u * FRAG * static_cast<uint32_t>(opA ? (t >> 16) : (t & 0xFFFF)) + op_run0;
  };
  uint32_t op_cur = op_base_of(ti);
  uint32_t aux_cur = wave < 2 ? scale_off(ti, 2) : bias_off(ti);
  const uint32_t aux_step = wave < 2 ? 2u * aux_lim : 0u;
  auto advance = [&]() {
    so = so == (F_NS - 1) * F_SLOT ? 0u : so + F_SLOT;
    if (++li == SPT) {
      li = 0;
      ++ji;
      ti = tnx;
      tnx = tile_at(ji + 1);
      op_cur = op_base_of(ti);
      aux_cur = wave < 2 ? scale_off(ti, 2) : bias_off(ti);
    } else {
      op_cur += 2u * op_gstride;
      aux_cur += aux_step;
    }
  };
  // The fused QKV epilogue's rotary factors (one tile per block; a tile with
  // Q / K columns and tables given): rows 64 g .. 64 g + 63 of the tile (the
  // rows of the waves with wm = g) of each table form a 16 KB piece, moved by
  // LDS-DMA (a load of a wave fills four 256-byte rows; rows past M read
  // zeros) in three parts into ring slots as they fall free: part 0 (cos and
  // sin of g = 0, cos of g = 3) and part 1 (cos and sin of g = 1, sin of
  // g = 3) take the places of the two padding stages issued during the
  // tile's last two stages, six loads per wave each (with the auxiliary load,
  // the usual seven); part 2 (cos and sin of g = 2) goes into the slot of
  // the last stage once the tile has ended.
  const bool qkv_rot = EPI == 2 && qa.cos != nullptr && F_BN * (ti & 0xFFFF) < 2 * (N / 3);   // uniform
  const int qkv_m0 = F_BM * (ti >> 16);
  auto qkv_table_dma = [&](int part, uint32_t slot_lds) {
    const int ln = fresh_lane();
    const uint32_t tbytes = static_cast<uint32_t>(M) * 256u;
    const int per = part < 2 ? 6 : 4;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      if (k < per) {
        const int q = per * wave + k;
        const int pc = q >> 4, c = q & 15;
        const bool is_sin = pc == 1 || (part == 1 && pc == 2);
        const int g = part == 2 ? 2 : (pc < 2 ? part : 3);
        const int row = qkv_m0 + 64 * g + 4 * c + (ln >> 4);
        const uint32_t voff = row < M ? static_cast<uint32_t>(row) * 256u + 16u * (ln & 15) : OOB;
        dma16(dma_rsrc(is_sin ? qa.sin : qa.cos, tbytes),
              __builtin_amdgcn_readfirstlane(slot_lds + 16384u * pc + 1024u * c), voff);
      }
    }
  };
  auto issue = [&]() {
    const bool live = ji < my_tiles;
    const uint32_t blds = __builtin_amdgcn_readfirstlane(bias_lds + 512u * static_cast<uint32_t>(ji & 1));
    if (live && 2 * (li + 2) <= G) {
      const int ln = fresh_lane();
      dma16x3(op_rs, __builtin_amdgcn_readfirstlane(op_lds + so), op_cur + 16u * ln);
      dma16x3(op_rs, __builtin_amdgcn_readfirstlane(op_lds + so + F_HALF), op_cur + op_gstride + 16u * ln);
      if (wave < 2)
        dma16(aux_rs, __builtin_amdgcn_readfirstlane(aux_lds + so),
              aux_cur + static_cast<uint32_t>(ln >> 5) * aux_lim + 16u * (ln & 31));
      else
        dma4(aux_rs, blds, aux_cur + 4u * ln);
      advance();
      return;
    }
    // per-lane parts of the addresses (the rest is wave-uniform); rows past
    // M or N lie past the end of their buffer and read as zero
    const int ln = fresh_lane();
    const uint32_t l16 = 16u * ln;
    const int tmi = ti >> 16, tni = ti & 0xFFFF;
    if (EPI == 2 && qkv_rot && !live && li < 2) {
      qkv_table_dma(li, __builtin_amdgcn_readfirstlane(ring0 + so));
    } else if (li < GS || !live) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int g = 2 * li + hh;
        const uint32_t base = __builtin_amdgcn_readfirstlane(
            live && g < G ? op_base_of(ti) + static_cast<uint32_t>(g) * op_gstride : OOB);
        dma16x3(op_rs, __builtin_amdgcn_readfirstlane(op_lds + so + F_HALF * hh), base + l16);
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ch = 2 * (li - GS) + hh;                     // rank chunk; >= NR: padding
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const int q = 3 * wave + i;
          const bool isla = q < 16;
          const int row0 = isla ? F_BM * tmi + 16 * q : F_BN * tni + 32 * (q - 16);
          const uint32_t base = __builtin_amdgcn_readfirstlane(
              ch < NR ? (static_cast<uint32_t>(row0) * rank + 16u * ch) * (isla ? 4u : 2u) : OOB);
          const uint32_t lds = __builtin_amdgcn_readfirstlane(op_lds + 1024 * i + so + F_HALF * hh);
          if (isla)
            dma16(la_rs, lds, base + static_cast<uint32_t>(ln >> 2) * static_cast<uint32_t>(rank * 4) + 16u * (ln & 3));
          else
            dma16(lu_rs, lds, base + static_cast<uint32_t>(ln >> 1) * static_cast<uint32_t>(rank * 2) + 16u * (ln & 1));
        }
      }
    }
    if (wave < 2) {
      // scales of the following stage: groups 2 (li + 1), + 1 of this tile,
      // or groups 0, 1 of the next tile
      const int lnext = li + 1;
      const bool same = live && lnext < GS, nxt = live && lnext == SPT && ji + 1 < my_tiles;
      scale_load(__builtin_amdgcn_readfirstlane(aux_lds + so), same ? ti : tnx, same ? 2 * lnext : (nxt ? 0 : -1));
    } else {
      dma4(aux_rs, blds, (live ? bias_off(ti) : OOB) + 4u * ln);
    }
    advance();
  };
  // Thread t converts raw scales t and t + 512 of slot `slot` to fp32.  No
  // bounds: rows M .. Mp - 1 hold zero scales; rows and columns past the
  // operands read other groups' scales or zeros, and their outputs are
  // never stored.
  auto convert_scales = [&](int slot, int buf) {
    int t = tid;
    asm volatile("" : "+v"(t));
    const _Float16* raw = reinterpret_cast<const _Float16*>(&ring[slot][F_SC]);
    const float lo = static_cast<float>(raw[t]), hi = static_cast<float>(raw[t + F_THREADS]);
    conv[buf][t] = lo;
    conv[buf][t + F_THREADS] = hi;
  };

  v16f acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][t][e] = 0.f;

  // per-lane LDS byte offsets in a group half of a slot
  const uint32_t a_off = (2 * wm) * FRAG + lane16;             // + a * FRAG; dwords 4-5 at + 1024 - 8 lane
  const uint32_t b_off = F_A + (4 * wn) * FRAG + lane16;
  const v16f zero = {};

  // Stage 0's scales into slot F_NS - 1's scale area (free until stage
  // F_NS - 1 is issued); then stages 0 .. F_NS - 2.
  if (wave < 2) scale_load(__builtin_amdgcn_readfirstlane(aux_lds + (F_NS - 1) * F_SLOT), ti, 0);
#pragma unroll
  for (int k = 0; k < F_NS - 1; ++k) issue();
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(F_DMA * (F_NS - 2)));   // stage 0's scales and stage 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  convert_scales(F_NS - 1, 0);

  int s = 0;                 // stage index in the block's sequence
  int sc = 0;                // its slot
  int since_end = 8;         // stages since the last tile end (its stores outstanding if < F_NS - 1)
  // Top of stage s: its loads landed (stage s + 1 may be in flight, and the
  // stores of a tile that ended in the last F_NS - 1 stages); the barrier
  // publishes them; then stage s + 2 is issued and stage s + 1's scales
  // converted.
  auto stage_top = [&]() {
    if (since_end < F_NS - 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(F_DMA * (F_NS - 2) + F_STORES));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(F_DMA * (F_NS - 2)));
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
    if (since_end < F_NS - 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(F_DMA * (F_NS - 2) + F_STORES));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(F_DMA * (F_NS - 2)));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto stage_issue = [&]() {
    issue();
    convert_scales(sc, (s + 1) & 1);
  };
  auto stage_end = [&]() {
    ++s;
    sc = sc == F_NS - 1 ? 0 : sc + 1;
    ++since_end;
  };

  // The chain's epilogue (one tile per block): once every load of the ring
  // has landed, the ring holds the output tile as bf16 (E1); each thread then
  // takes two (row, group of 64) pairs through tanh-GELU, the next layer's
  // smoothing and INT4 quantizer -- the arithmetic of kernel 1 -- writes
  // their codes into the 6-bit containers and their fp16 scales, and puts
  // bf16(x_hat) back in place (E2); the block then stages the tile's
  // 32-rank slice of L1 in the ring past the staging tile, and each wave
  // forms 32 rows of the tile's partial down projection, bf16(x_hat)
  // [256 x 256] L1 slice, on bf16 MFMA with both operands from LDS (E3).  Rows M .. Mp - 1 get zero codes and scales, as kernel 1
  // writes them; rows and groups past the operands are not written.
  auto chain_epilogue = [&](int tt) {
    if constexpr (EPI == 1) {
      const int tmc = tt >> 16, tnc = tt & 0xFFFF;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      __syncthreads();
      unsigned char* T = &ring[0][0];
      float* si_s = &conv[0][0];
      {
        const int ln = fresh_lane();
        const int lc = ln & 31, lh = ln >> 5;
        const uint2 bu = *reinterpret_cast<const uint2*>(&bias_ring[0][128 * wn + 4 * lc]);
        const float bv[4] = {bf16_bits_to_f32(bu.x & 0xFFFFu), bf16_bits_to_f32(bu.x >> 16),
                             bf16_bits_to_f32(bu.y & 0xFFFFu), bf16_bits_to_f32(bu.y >> 16)};
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int e = 4 * b + i;
              const int rl = 64 * wm + 32 * a + 8 * b + 4 * lh + i;
              *reinterpret_cast<uint2*>(T + rl * C_TS + 2 * (128 * wn + 4 * lc)) =
                  make_uint2(bf16x2_bits(acc[a][0][e] + bv[0], acc[a][1][e] + bv[1]),
                             bf16x2_bits(acc[a][2][e] + bv[2], acc[a][3][e] + bv[3]));
            }
        if (tid < F_BN) {
          const int k = F_BN * tnc + tid;
          si_s[tid] = k < N ? ca.smooth_inv[k] : 0.f;
        }
      }
      __syncthreads();
      // The tile's slice of L1^T, ranks rc .. rc + 31 by its 256 k, goes to
      // the ring past the staging tile (row stride C_TS, so that the 16
      // ranks one MFMA operand read touches fall on distinct banks): two
      // coalesced 16-byte chunks per thread, ranks past the rank and k past
      // N as zeros.  The first slice's loads are issued after E2's loop, so
      // their latency overlaps the barrier that closes E2.
      unsigned char* Ls = T + F_BM * C_TS;
      auto l1_load = [&](int rc, uint4 (&v)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int f = tid + F_THREADS * j;
          const int rr = rc + (f >> 5), kg = F_BN * tnc + 8 * (f & 31);
          const bool ok = rr < ca.rank && kg < N;
          v[j] = *reinterpret_cast<const uint4*>(ca.lora_down + static_cast<size_t>(ok ? rr : 0) * N + (ok ? kg : 0));
          if (!ok) v[j] = make_uint4(0, 0, 0, 0);
        }
      };
      auto l1_store = [&](const uint4 (&v)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int f = tid + F_THREADS * j;
          *reinterpret_cast<uint4*>(Ls + (f >> 5) * C_TS + 16 * (f & 31)) = v[j];
        }
      };
      uint4 lv[2];
      const int RBd = (M + 31) >> 5, Mpd = RBd << 5;
      const int Gd = N / GROUP;
      // units of 32 values: (row, group, half hh) = p >> 3, (p >> 1) & 3, p & 1,
      // p = tid + 512 k; lanes tid and tid ^ 1 hold the two halves of a
      // group and exchange their absmax; a unit's 32 codes are exactly one
      // lane of the group's 6-bit container fragment
#pragma unroll 1
      for (int k4 = 0; k4 < 4; ++k4) {
        const int p = tid + F_THREADS * k4;
        const int rl = p >> 3, g = (p >> 1) & 3, hh = p & 1;
        const int row = F_BM * tmc + rl;
        const int gd = 4 * tnc + g;
        const bool live = gd < Gd && row < Mpd;               // uniform over the lane pair
        unsigned char* tr = T + rl * C_TS + 2 * (GROUP * g + 32 * hh);
        const float4* sp = reinterpret_cast<const float4*>(si_s + GROUP * g + 32 * hh);
        // every value is formed unconditionally (a per-value row test
        // compiles to one branch per value, which serializes the GELU's
        // exp2 and reciprocal); rows past M are zeroed through the scale
        float xh[32];
#pragma unroll
        for (int c8 = 0; c8 < 4; ++c8) {
          const uint4 u = *reinterpret_cast<const uint4*>(tr + 16 * c8);
          const float4 s0 = sp[2 * c8], s1 = sp[2 * c8 + 1];
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
          const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 8 * c8 + 2 * i;
            xh[j] = gelu_tanh(bf16_bits_to_f32(w[i] & 0xFFFFu)) * sv[2 * i];
            xh[j + 1] = gelu_tanh(bf16_bits_to_f32(w[i] >> 16)) * sv[2 * i + 1];
          }
        }
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(xh[j]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        // Rows M .. Mp - 1 (their staged values are the bias alone, finite):
        // scale 0 makes every code +0 below, as kernel 1 writes such rows.
        // Their bf16(x_hat) left in the staging tile only reaches the down
        // projection's rows past M, which are not stored.
        if (row >= M) amax = 0.f;
        const float s32 = amax / 7.0f;
        const _Float16 sh = static_cast<_Float16>(s32);
        const float sf = static_cast<float>(sh);
        const float rcp = (sf == 0.f) ? 0.f : 1.0f / sf;
        if (live) {
          // codes j = 0..31: even positions from the first source, odd from
          // the second; + 0.0f turns -0 into +0
          v16f ev, od;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            ev[i] = fminf(fmaxf(rintf(xh[2 * i] * rcp), -8.f), 7.f) + 0.0f;
            od[i] = fminf(fmaxf(rintf(xh[2 * i + 1] * rcp), -8.f), 7.f) + 0.0f;
          }
          typedef int v6i_ __attribute__((ext_vector_type(6)));
          const v6i_ pk = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, 1.0f);
          uint8_t* fr = ca.x_fp6 + (static_cast<size_t>(gd) * RBd + (row >> 5)) * FRAG;
          const int fl = (row & 31) + 32 * hh;
          *reinterpret_cast<uint4*>(fr + 16 * fl) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
          *reinterpret_cast<uint2*>(fr + 1024 + 8 * fl) = make_uint2(pk[4], pk[5]);
          if (hh == 0) ca.x_scales[static_cast<size_t>(gd) * Mpd + row] = sh;
        }
#pragma unroll
        for (int c8 = 0; c8 < 4; ++c8)
          *reinterpret_cast<uint4*>(tr + 16 * c8) =
              make_uint4(bf16x2_bits(xh[8 * c8], xh[8 * c8 + 1]), bf16x2_bits(xh[8 * c8 + 2], xh[8 * c8 + 3]),
                         bf16x2_bits(xh[8 * c8 + 4], xh[8 * c8 + 5]), bf16x2_bits(xh[8 * c8 + 6], xh[8 * c8 + 7]));
      }
      if (ca.rank > 0) l1_load(0, lv);
      __syncthreads();
      if (ca.rank > 0) {
        l1_store(lv);
        __syncthreads();
        // A = 8 bf16(x_hat) of row 32 w + l % 32 at k = 16 kk + 8 (l / 32);
        // B = the same k of the staged L1^T row (rank) rc + l % 32; D lane
        // l: rank rc + l % 32, rows 8 b + 4 (l / 32) + i of the wave's 32
        const int ln = fresh_lane();
        const int lc = ln & 31, lh = ln >> 5;
        const int rl = 32 * wave + lc;
#pragma unroll 1
        for (int rc = 0; rc < ca.rank; rc += 32) {
          if (rc > 0) {
            l1_load(rc, lv);
            __syncthreads();                                  // every wave is past the previous slice
            l1_store(lv);
            __syncthreads();
          }
          const int rr = rc + lc;
          v16f d = zero;
#pragma unroll 8
          for (int kk = 0; kk < F_BN / 16; ++kk) {
            const int kl = 16 * kk + 8 * lh;
            const v8bf av = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(T + rl * C_TS + 2 * kl));
            const v8bf bv = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(Ls + lc * C_TS + 2 * kl));
            d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, d, 0, 0, 0);
          }
          if (rr < ca.rank) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int row = F_BM * tmc + 32 * wave + 8 * b + 4 * lh + i;
                if (row < M)
                  ca.partials[(static_cast<size_t>(tnc) * M + row) * ca.rank + rr] = d[4 * b + i];
              }
          }
        }
      }
    }
  };

  // The QKV epilogue (one tile per block): bias into the accumulators, then
  // for a wave whose 128 columns are a Q or K head, per row the sum of
  // squares over the head (the lane's four columns, then the 32 lanes of its
  // half), the scale 1 / sqrt(sum / 128 + eps), the norm weights, and the
  // rotation.  Two thirds of the rotary factors are in the ring already
  // (parts 0 and 1 above); part 2 is loaded while the norms are formed.  A
  // lane's pairs are columns (4 c, 4 c + 1) and (4 c + 2, 4 c + 3) of the
  // head: factors 2 c and 2 c + 1 of its row, one 8-byte read per table (32
  // lanes read a row's 256 contiguous bytes) from its wave's pieces.  Tiles whose
  // columns are all V (2 H 128 is a multiple of 256, so a tile is all Q / K
  // or all V) only add the bias.
  auto qkv_epilogue = [&](int tt, const float (&bv)[4]) {
    if constexpr (EPI == 2) {
      const int HD = N / 3;
      const int cw = F_BN * (tt & 0xFFFF) + 128 * wn;
      // slots of the tile's stages SPT (part 0), SPT + 1 (part 1), SPT - 1 (part 2)
      const uint32_t sA = static_cast<uint32_t>(SPT % F_NS) * F_SLOT;
      const uint32_t sB = static_cast<uint32_t>((SPT + 1) % F_NS) * F_SLOT;
      const uint32_t sC = static_cast<uint32_t>((SPT - 1) % F_NS) * F_SLOT;
      if (qkv_rot) {
        // every wave is past its reads of the last stage's slot (their values
        // are in the accumulators); parts 0 and 1 may still be landing
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        qkv_table_dma(2, __builtin_amdgcn_readfirstlane(ring0 + sC));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[a][t][e] += bv[t];
      const bool qk = cw < 2 * HD;                            // wave-uniform
      const int ln = fresh_lane();
      const int lc = ln & 31, lh = ln >> 5;
      if (qk) {
        const uint16_t* g = cw < HD ? qa.gq : qa.gk;
        const uint2 gu = *reinterpret_cast<const uint2*>(g + 4 * lc);
        const float g4[4] = {bf16_bits_to_f32(gu.x & 0xFFFFu), bf16_bits_to_f32(gu.x >> 16),
                             bf16_bits_to_f32(gu.y & 0xFFFFu), bf16_bits_to_f32(gu.y >> 16)};
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float ss = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t) ss = __builtin_fmaf(acc[a][t][e], acc[a][t][e], ss);
            ss = sum32(ss);
            // hardware reciprocal square root (1 ulp)
            const float scale = __builtin_amdgcn_rsqf(ss * (1.0f / Q_HEAD) + qa.eps);
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[a][t][e] = acc[a][t][e] * scale * g4[t];
          }
      }
      if (qkv_rot) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const uint32_t cb = wm == 0 ? sA : (wm == 1 ? sB : (wm == 2 ? sC : sA + 32768u));
        const uint32_t sb = wm == 0 ? sA + 16384u : (wm == 1 ? sB + 16384u : (wm == 2 ? sC + 16384u : sB + 32768u));
        const unsigned char* tc = &ring[0][0] + cb;
        const unsigned char* ts = &ring[0][0] + sb;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int rl = 32 * a + 8 * (e >> 2) + 4 * lh + (e & 3);   // row within the wave's 64
            const float2 cs = *reinterpret_cast<const float2*>(tc + rl * 256 + 8 * lc);
            const float2 sn = *reinterpret_cast<const float2*>(ts + rl * 256 + 8 * lc);
            const float o0 = acc[a][0][e], o1 = acc[a][1][e], o2 = acc[a][2][e], o3 = acc[a][3][e];
            acc[a][0][e] = o0 * cs.x - o1 * sn.x;
            acc[a][1][e] = o1 * cs.x + o0 * sn.x;
            acc[a][2][e] = o2 * cs.y - o3 * sn.y;
            acc[a][3][e] = o3 * cs.y + o2 * sn.y;
          }
      }
    }
  };

  for (int j = 0; j < my_tiles; ++j) {
    const int tt = __builtin_amdgcn_readfirstlane(tiles[j]);
    const int mw = F_BM * (tt >> 16) + 64 * wm, cw = F_BN * (tt & 0xFFFF) + 128 * wn;   // wave-uniform

    // ---- the tile's groups: P_g on the 6-bit MFMA, then dequantization ----
    for (int l = 0; l < GS; ++l, stage_end()) {
      // (the chain's epilogue leaves no registers for the early reads)
      if constexpr (EPI == 1) stage_top();
      else stage_wait();
      // The stage's 16 tiles (two groups x 8) in one sequence u = 0..15:
      // group u / 8, then (n tile 0, m tile 0), (0, 1), (1, 0), ...  A
      // weight fragment serves two consecutive tiles and is read one tile
      // pair ahead; the second group's first fragments are read right after
      // the MFMA that last uses the first group's.  A tile's row scales are
      // read from LDS four at a time as it is dequantized (two distinct
      // addresses per read: broadcast).  The MFMA of tile u + 1 is issued
      // before tile u is dequantized (results in a ring of two).  When K / 64
      // is odd the last stage's second group is all zero codes and zero
      // scales and adds nothing.
      const unsigned char* sl = ring[sc];
      const float* cv = conv[s & 1];
      auto rd_frag = [&](uint32_t off) {
        const uint4 lo = *reinterpret_cast<const uint4*>(sl + off);
        const uint2 hi = *reinterpret_cast<const uint2*>(sl + off + 1024 - 8 * lane);
        return v8i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                   static_cast<int>(hi.x), static_cast<int>(hi.y), 0, 0};
      };
      v8i afr[2];
      afr[0] = rd_frag(a_off);
      afr[1] = rd_frag(a_off + FRAG);
      v8i bfr[4];
      bfr[0] = rd_frag(b_off);
      if constexpr (EPI != 1) stage_issue();
      v16f dr[2];
      float swv[4];
#pragma unroll
      for (int u = 0; u < 17; ++u) {
        if (u < 16) {
          const int hg = u >> 3, t = (u >> 1) & 3, a = u & 1;
          if (a == 0 && t < 3) bfr[t + 1] = rd_frag(F_HALF * hg + b_off + (t + 1) * FRAG);
          // cbsz = blgp = 3: both operands E3M2; E8M0 scales 127 (= 1)
          dr[u & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afr[a], bfr[t], zero, 3, 3, 0, 127, 0, 127);
          if (u == 7) {
            afr[0] = rd_frag(F_HALF + a_off);
            afr[1] = rd_frag(F_HALF + a_off + FRAG);
            bfr[0] = rd_frag(F_HALF + b_off);
          }
        }
        if (u > 0) {
          const int v = u - 1, hv = v >> 3, t = (v >> 1) & 3, a = v & 1;
          if ((v & 7) == 0) {
            const float4 sw = *reinterpret_cast<const float4*>(cv + F_GPS * F_BM + F_BN * hv + 128 * wn + 4 * c);
            swv[0] = sw.x; swv[1] = sw.y; swv[2] = sw.z; swv[3] = sw.w;
          }
          const float* sxp = cv + F_BM * hv + 64 * wm + 4 * h;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float4 s4 = *reinterpret_cast<const float4*>(sxp + 32 * a + 8 * b);
            const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int e = 4 * b + i;
              acc[a][t][e] = __builtin_fmaf(dr[v & 1][e] * sv[i], swv[t], acc[a][t][e]);
            }
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
        const unsigned char* sl = ring[sc] + F_HALF * hh;
        // A = bf16(lora_act) rows (lane row l % 32 of m tile a, ranks
        // 8h .. 8h + 7 of the chunk), B = lora_up rows (columns
        // n_w + 4 (l % 32) + t, the same ranks); products into a ring of
        // two, added like the group results (the accumulators stay single
        // registers for the dequantization FMAs)
        const int ln = fresh_lane();
        const int lc = ln & 31, lh = ln >> 5;
        v8bf la[2], lu[4];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const float4* p = reinterpret_cast<const float4*>(sl + F_LA + (64 * wm + 32 * a + lc) * 64 + 32 * lh);
          const float4 v0 = p[0], v1 = p[1];
          const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          la[a] = pack_bf16x8(v);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
          lu[t] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(sl + F_LU + (128 * wn + 4 * lc + t) * 32 + 16 * lh));
        v16f dr[2];
#pragma unroll
        for (int u = 0; u < 9; ++u) {
          if (u < 8) dr[u & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[u >> 2], lu[u & 3], zero, 0, 0, 0);
          if (u > 0) {
            const int v = u - 1;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[v >> 2][v & 3][e] += dr[v & 1][e];
          }
        }
      }
    }

    // ---- end of the tile, after its last stage ----
    if constexpr (EPI == 1) {
      chain_epilogue(tt);
    } else {
      // The bias ring entry of tile j is rewritten only by the stages of
      // tile j + 2, issued after the next barrier.
      // end of the tile: bias, rounding, store.  The lane holds rows
      // mw + 32 a + 8 b + 4 h + i and columns cw + 4 c .. + 3; rows past M
      // fall past the end of y, columns past N (N % 8 == 0: a lane's four
      // are all in or all out) are sent past it.
      const int ln = fresh_lane();
      const int lc = ln & 31, lh = ln >> 5;
      const uint2 bu = *reinterpret_cast<const uint2*>(&bias_ring[j & 1][128 * wn + 4 * lc]);
      const float bv[4] = {bf16_bits_to_f32(bu.x & 0xFFFFu), bf16_bits_to_f32(bu.x >> 16),
                           bf16_bits_to_f32(bu.y & 0xFFFFu), bf16_bits_to_f32(bu.y >> 16)};
      if constexpr (EPI == 2) qkv_epilogue(tt, bv);
      // one per-lane base (row mw + 4 h, columns cw + 4 c); each store adds
      // its wave-uniform row offset.  A base past the end stays past it
      // (y is under 2 GiB, the added offsets under 32 rows).
      const uint32_t vbase = 4 * lc < N - cw
                                 ? ((static_cast<uint32_t>(mw) + 4u * lh) * static_cast<uint32_t>(N) +
                                    static_cast<uint32_t>(cw) + 4u * lc) * ELEM
                                 : OOB;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * b + i;
            const uint32_t off = vbase + static_cast<uint32_t>(32 * a + 8 * b + i) * static_cast<uint32_t>(N) * ELEM;
            // (the QKV epilogue has added the bias already)
            float o[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) o[t] = EPI == 2 ? acc[a][t][e] : acc[a][t][e] + bv[t];
            if (OUT_F32) {
              const v4f ov = v4f{o[0], o[1], o[2], o[3]};
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, ov), y_rs, off, 0, 0);
            } else {
              typedef int v2i_ __attribute__((ext_vector_type(2)));
              const v2i_ ov = v2i_{static_cast<int>(bf16x2_bits(o[0], o[1])), static_cast<int>(bf16x2_bits(o[2], o[3]))};
              __builtin_amdgcn_raw_buffer_store_b64(ov, y_rs, off, 0, 0);
            }
          }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[a][t][e] = 0.f;
      since_end = 0;
    }
  }
  // drain the padding loads issued past the last stage (and the stores)
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
}

// lora_act = the column slices' partial down projections summed in slice
// order (the chain's second pass); four ranks per thread.  The loads of 16
// slices go out before their sums (the sum stays in slice order), and
// 64-thread blocks spread the few outputs over every CU: the pass is a
// read of the partials, bound by how many loads are in flight.
constexpr int R_THREADS = 64;
constexpr int R_BATCH = 16;
__global__ __launch_bounds__(R_THREADS) void k_partials_reduce(const float4* __restrict__ partials, int S,
                                                             size_t n4, float4* __restrict__ lora_act) {
  const size_t i = static_cast<size_t>(blockIdx.x) * R_THREADS + threadIdx.x;
  if (i >= n4) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int s = 0;
  for (; s + R_BATCH <= S; s += R_BATCH) {
    float4 v[R_BATCH];
#pragma unroll
    for (int u = 0; u < R_BATCH; ++u) v[u] = partials[static_cast<size_t>(s + u) * n4 + i];
#pragma unroll
    for (int u = 0; u < R_BATCH; ++u) {
      acc.x += v[u].x;
      acc.y += v[u].y;
      acc.z += v[u].z;
      acc.w += v[u].w;
    }
  }
  for (; s < S; ++s) {
    const float4 v = partials[static_cast<size_t>(s) * n4 + i];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  lora_act[i] = acc;
}

// The no-allocation variant of the MLP chain keeps its partial down
// projections here instead of in a caller's workspace: one copy per device,
// held until the process ends.  Host code uses only the per-device address
// from hipGetSymbolAddress, never this name.
constexpr size_t CHAIN_SCRATCH_BYTES = SVDQ_CHAIN_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[CHAIN_SCRATCH_BYTES];

}  // namespace

namespace svdq {

int launch_gemm_w4a4_fp6(const void* x_fp6, const void* x_scales, const void* w_fp6, const void* w_scales,
                         const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K, int rank,
                         int out_dtype, void* y, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int tiles = ((M + F_BM - 1) / F_BM) * ((N + F_BN - 1) / F_BN);
  // one block per CU, a multiple of 8 (the XCD count) so that a block's
  // tiles stay on its XCD; never more blocks than tiles
  const int cus = device_cu_count() & ~7;
  const int grid = tiles < cus ? tiles : (cus > 0 ? cus : tiles);
  if ((tiles + grid - 1) / grid > F_MAX_TILES) return SVDQ_ERR_UNSUPPORTED_SHAPE;
#define SVDQ_K2F(OF)                                                                                          \
  hipLaunchKernelGGL((k_gemm_w4a4_fp6<OF, 0>), dim3(grid), dim3(F_THREADS), 0, st,                            \
                     static_cast<const uint8_t*>(x_fp6), static_cast<const _Float16*>(x_scales),              \
                     static_cast<const uint8_t*>(w_fp6), static_cast<const _Float16*>(w_scales), lora_act,    \
                     static_cast<const uint16_t*>(lora_up), static_cast<const uint16_t*>(bias), M, N, K, rank, y, \
                     ChainArgs{}, QkvArgs6{})
  if (out_dtype == SVDQ_OUT_F32) SVDQ_K2F(1);
  else SVDQ_K2F(0);
#undef SVDQ_K2F
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

int launch_gemm_w4a4_fp6_qkv(const void* x_fp6, const void* x_scales, const void* w_fp6, const void* w_scales,
                             const float* lora_act, const void* lora_up, const void* bias, const void* norm_q,
                             const void* norm_k, const float* rope_cos, const float* rope_sin, float eps, int M, int N,
                             int K, int rank, int out_dtype, void* y, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int tiles = ((M + F_BM - 1) / F_BM) * ((N + F_BN - 1) / F_BN);
  const QkvArgs6 qa{static_cast<const uint16_t*>(norm_q), static_cast<const uint16_t*>(norm_k), rope_cos, rope_sin,
                    eps};
  // one tile per block: the ring is free for the rotary tables at its end
#define SVDQ_K2Q(OF)                                                                                          \
  hipLaunchKernelGGL((k_gemm_w4a4_fp6<OF, 2>), dim3(tiles), dim3(F_THREADS), 0, st,                           \
                     static_cast<const uint8_t*>(x_fp6), static_cast<const _Float16*>(x_scales),              \
                     static_cast<const uint8_t*>(w_fp6), static_cast<const _Float16*>(w_scales), lora_act,    \
                     static_cast<const uint16_t*>(lora_up), static_cast<const uint16_t*>(bias), M, N, K, rank, y, \
                     ChainArgs{}, qa)
  if (out_dtype == SVDQ_OUT_F32) SVDQ_K2Q(1);
  else SVDQ_K2Q(0);
#undef SVDQ_K2Q
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

size_t chain_scratch_bytes() { return CHAIN_SCRATCH_BYTES; }

int chain_scratch(void** ptr) {
  // address of the current device's copy, looked up once per device with
  // that device current
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SVDQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SVDQ_ERR_HIP;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return SVDQ_OK;
}

int launch_mlp_chain_fp6(const void* x_fp6, const void* x_scales, const void* w_fp6, const void* w_scales,
                         const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K, int rank,
                         const float* smooth_inv_dn, const void* lora_down_dn, int rank_dn, void* x_fp6_dn,
                         void* x_scales_dn, float* lora_act_dn, float* partials, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int tiles = ((M + F_BM - 1) / F_BM) * ((N + F_BN - 1) / F_BN);
  ChainArgs ca{smooth_inv_dn, static_cast<const uint16_t*>(lora_down_dn), rank_dn, static_cast<uint8_t*>(x_fp6_dn),
               static_cast<_Float16*>(x_scales_dn), partials};
  // one tile per block: the ring is free for the staging tile at its end
  hipLaunchKernelGGL((k_gemm_w4a4_fp6<0, 1>), dim3(tiles), dim3(F_THREADS), 0, st,
                     static_cast<const uint8_t*>(x_fp6), static_cast<const _Float16*>(x_scales),
                     static_cast<const uint8_t*>(w_fp6), static_cast<const _Float16*>(w_scales), lora_act,
                     static_cast<const uint16_t*>(lora_up), static_cast<const uint16_t*>(bias), M, N, K, rank,
                     nullptr, ca, QkvArgs6{});
  if (rank_dn > 0) {
    const int S = (N + F_BN - 1) / F_BN;
    const size_t n4 = static_cast<size_t>(M) * rank_dn / 4;
    hipLaunchKernelGGL(k_partials_reduce, dim3(static_cast<unsigned>((n4 + R_THREADS - 1) / R_THREADS)),
                       dim3(R_THREADS), 0, st,
                       reinterpret_cast<const float4*>(partials), S, n4, reinterpret_cast<float4*>(lora_act_dn));
  }
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

}  // namespace svdq
