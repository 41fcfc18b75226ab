// Device helpers shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int GROUP = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return static_cast<uint32_t>(__builtin_bit_cast(unsigned short, b));
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two fp32 -> one dword of bf16 bits (a in the low half), round to nearest
// even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

__device__ __forceinline__ v8bf pack_bf16x8(const float* v) {
  const uint4 u = make_uint4(bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3]), bf16x2_bits(v[4], v[5]),
                             bf16x2_bits(v[6], v[7]));
  return __builtin_bit_cast(v8bf, u);
}

// Tanh-form GELU, 0.5 x (1 + tanh u) with u = sqrt(2/pi) (x + 0.044715 x^3),
// evaluated through the identity 0.5 (1 + tanh u) = 1 / (1 + e^(-2u)):
// x / (1 + 2^(x (c1 + c3 x^2))), c1 = -2 sqrt(2/pi) / ln 2, c3 = 0.044715 c1.
// One hardware exp2 and one reciprocal (about 1 ulp each) in place of a
// tanh, and no cancellation in 1 + tanh u for negative x (the tanh form
// loses up to ~1e-4 relative there in fp32; this one stays near 1e-6).
// Large negative x gives e = +inf and a signed zero.
__device__ __forceinline__ float gelu_tanh(float x) {
  constexpr float c1 = -2.302208198144325f;
  constexpr float c3 = -0.1029432395800235f;
  const float e = __builtin_amdgcn_exp2f(x * (c1 + c3 * (x * x)));
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// Eight packed E2M1 codes: every -0 (nibble 1000b) becomes +0.  A nibble's
// low three bits plus 7 carry into its bit 3 exactly when they are nonzero.
__device__ __forceinline__ uint32_t e2m1_clear_neg_zero(uint32_t x) {
  const uint32_t nz = ((x & 0x77777777u) + 0x77777777u) & 0x88888888u;
  return x ^ (x & 0x88888888u & ~nz);
}

// Map the linear block index to an output tile so that the blocks of one
// XCD (the hardware deals blocks round-robin over 8 XCDs) cover a compact
// band of rows and share A panels and B panels in their L2.
__device__ __forceinline__ void xcd_tile(int nM, int nN, int& tm, int& tn) {
  const int nb = nM * nN;
  const int b = blockIdx.x;
  int t = b;
  if ((nb & 7) == 0) t = (b & 7) * (nb >> 3) + (b >> 3);
  constexpr int GM = 4;
  const int per = GM * nN;
  const int grp = t / per;
  const int first = grp * GM;
  const int gm = min(GM, nM - first);
  const int r = t - grp * per;
  tm = first + r % gm;
  tn = r / gm;
}

// Buffer descriptor (raw, stride 0) in four scalar registers: byte base,
// size in bytes (accesses at or past it read zeros), default format word.
struct DmaRsrc {
  v4i w;
};
__device__ __forceinline__ DmaRsrc dma_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  DmaRsrc r;
  r.w[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xFFFFFFFFu));
  r.w[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xFFFFu));
  r.w[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r.w[3] = 0x00020000;
  return r;
}

// LDS-DMA buffer loads: lane l's `size` bytes at byte offset voff of the
// buffer land at LDS address lds_addr + size * l.  Issued from inline
// assembly so that the compiler does not treat the pending LDS writes as
// aliasing every later LDS read (it would wait for all of them); the kernel
// waits for them itself with s_waitcnt vmcnt before the barrier that
// publishes a stage.  s_nop 4 covers the wait states after M0 and scalar
// register writes that a buffer load reading them needs.  No register is
// written, so nothing stays in flight towards a register.
__device__ __forceinline__ void dma16(const DmaRsrc& r, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(r.w) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const DmaRsrc& r, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(r.w) : "memory", "m0");
}

// s_waitcnt immediate: vmcnt = v (0..63), expcnt and lgkmcnt = 0.
constexpr int waitcnt_vm_lgkm0(int v) { return (v & 0xF) | ((v >> 4) << 14) | (0x0 << 4) | (0x0 << 8); }
// s_waitcnt immediate: vmcnt = v (0..63) only; expcnt and lgkmcnt at their
// maxima (no wait).
constexpr int waitcnt_vm(int v) { return (v & 0xF) | ((v >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

}  // namespace
