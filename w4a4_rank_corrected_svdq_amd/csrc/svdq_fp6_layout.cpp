// Host side of the 6-bit operand container of the INT4 layer (see
// svdq_fp6_kernels.hip): the E3M2 encoding of the integer codes -8 .. 7 and
// the fragment layout kernel 2 reads.  Preparation stores the weight codes
// as nibbles (the layer's 4-bit format); svdq_pack_fp6_operand re-packs
// them once for the device.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "svdq.h"
#include "svdq_internal.h"

namespace {

constexpr int kFrag = 1536;

// E3M2 bit pattern of the integer q, |q| <= 8: sign in bit 5, biased
// exponent (bias 3) in bits 4..2, two mantissa bits; 0 is +0.
uint8_t e3m2_of_int(int q) {
  static const uint8_t mag[9] = {0x00, 0x0C, 0x10, 0x12, 0x14, 0x15, 0x16, 0x17, 0x18};
  return static_cast<uint8_t>((q < 0 ? 0x20 : 0) | mag[q < 0 ? -q : q]);
}

int nibble_code(const uint8_t* row, int k) {
  const int v = (row[k >> 1] >> (4 * (k & 1))) & 0xF;
  return v >= 8 ? v - 16 : v;
}

int64_t host_threads() {
  const unsigned hc = std::thread::hardware_concurrency();
  return std::max<int64_t>(1, std::min<int64_t>(hc ? hc : 4, 64));
}

int64_t row_blocks(int64_t rows, int layout) {
  return layout == SVDQ_FP6_WEIGHTS ? 4 * ((rows + 127) / 128) : (rows + 31) / 32;
}

}  // namespace

extern "C" int svdq_fp6_operand_bytes(int rows, int K, int layout, size_t* bytes_out) {
  if (!bytes_out || rows < 0 || K <= 0) return SVDQ_ERR_INVALID_ARG;
  if (layout != SVDQ_FP6_ACTIVATIONS && layout != SVDQ_FP6_WEIGHTS) return SVDQ_ERR_INVALID_ARG;
  if (K % SVDQ_GROUP != 0) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  *bytes_out = static_cast<size_t>(K / SVDQ_GROUP) * static_cast<size_t>(row_blocks(rows, layout)) * kFrag;
  return SVDQ_OK;
}

extern "C" int svdq_pack_fp6_operand(const uint8_t* codes, int rows, int K, int layout, uint8_t* out) {
  size_t bytes = 0;
  const int st = svdq_fp6_operand_bytes(rows, K, layout, &bytes);
  if (st != SVDQ_OK) return st;
  if (!out || (rows > 0 && !codes)) return SVDQ_ERR_INVALID_ARG;
  const int64_t RB = row_blocks(rows, layout);
  const int G = K / SVDQ_GROUP;
  const int64_t rowb = K / 2;
  // One task per (group, row block): fragment lane l = r + 32 h takes the
  // row that row block's slot r holds and k = 64 g + 32 h + j.
  auto fill = [&](int64_t f0, int64_t f1) {
    for (int64_t f = f0; f < f1; ++f) {
      const int g = static_cast<int>(f / RB);
      const int64_t rb = f % RB;
      uint8_t* frag = out + f * kFrag;
      for (int l = 0; l < 64; ++l) {
        const int r = l & 31, h = l >> 5;
        int64_t row;
        if (layout == SVDQ_FP6_WEIGHTS) row = 128 * (rb / 4) + 4 * r + (rb % 4);
        else row = 32 * rb + r;
        uint32_t w[6] = {0, 0, 0, 0, 0, 0};
        if (row < rows) {
          const uint8_t* src = codes + row * rowb;
          for (int j = 0; j < 32; ++j) {
            const uint64_t c = e3m2_of_int(nibble_code(src, 64 * g + 32 * h + j));
            const int bit = 6 * j;
            const uint64_t v = c << (bit & 31);
            w[bit >> 5] |= static_cast<uint32_t>(v);
            if ((bit & 31) > 26) w[(bit >> 5) + 1] |= static_cast<uint32_t>(v >> 32);
          }
        }
        std::memcpy(frag + 16 * l, w, 16);
        std::memcpy(frag + 1024 + 8 * l, w + 4, 8);
      }
    }
  };
  const int64_t nf = static_cast<int64_t>(G) * RB;
  const int64_t nt = std::max<int64_t>(1, std::min<int64_t>(host_threads(), nf / 64));
  std::vector<std::thread> pool;
  for (int64_t t = 0; t < nt; ++t) pool.emplace_back(fill, nf * t / nt, nf * (t + 1) / nt);
  for (auto& th : pool) th.join();
  return SVDQ_OK;
}
