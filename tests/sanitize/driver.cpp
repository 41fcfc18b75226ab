// Host driver for the sanitizer build: runs the library's host preparation
// (INT4, MXFP4, AWQ, the 6-bit operand packer) on small ragged shapes and
// every argument check of the C ABI, under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Prints "SANITIZE OK" when every status is the
// expected one; the sanitizers abort the process on the first finding.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "svdq.h"

namespace svdq { extern int g_launches; }

static int g_fail = 0;
#define EXPECT(cond)                                                          \
  do {                                                                        \
    if (!(cond)) { std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #cond); ++g_fail; } \
  } while (0)

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static double uniform() {
  g_rng ^= g_rng << 13; g_rng ^= g_rng >> 7; g_rng ^= g_rng << 17;
  return (g_rng >> 11) * (1.0 / 9007199254740992.0);
}
static double normal() {
  const double u = uniform() + 1e-300, v = uniform();
  return std::sqrt(-2.0 * std::log(u)) * std::cos(6.283185307179586 * v);
}
static uint16_t bf16_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
static std::vector<uint16_t> bf16_matrix(size_t n, double scale) {
  std::vector<uint16_t> v(n);
  for (auto& e : v) e = bf16_bits(static_cast<float>(normal() * scale));
  return v;
}

static void int4_prepare(int K, int N, int rank, float alpha, int power_iters, bool given_factors) {
  auto w = bf16_matrix(static_cast<size_t>(N) * K, 0.02);
  std::vector<float> a(K);
  for (auto& e : a) e = static_cast<float>(std::fabs(normal()) * 3.0 + 0.1);
  size_t bytes = 0;
  EXPECT(svdq_prepared_bytes(K, N, rank, 64, &bytes) == SVDQ_OK && bytes > 0);
  std::vector<float> si(K);
  std::vector<uint8_t> wc(static_cast<size_t>(N) * K / 2);
  std::vector<uint16_t> ws(static_cast<size_t>(K / 64) * N), ld(static_cast<size_t>(rank) * K),
      lu(static_cast<size_t>(N) * rank);
  std::vector<double> sigma(rank > 0 ? rank : 1);
  std::vector<uint16_t> ld_in, lu_in;
  if (given_factors) {
    ld_in = bf16_matrix(static_cast<size_t>(rank) * K, 0.05);
    lu_in = bf16_matrix(static_cast<size_t>(N) * rank, 0.05);
  }
  const int st = svdq_prepare_weights_ex(w.data(), K, N, a.data(), alpha, rank, 64,
                                         given_factors ? ld_in.data() : nullptr,
                                         given_factors ? lu_in.data() : nullptr, power_iters, 1234u, si.data(),
                                         wc.data(), ws.data(), rank ? ld.data() : nullptr,
                                         rank ? lu.data() : nullptr, sigma.data());
  EXPECT(st == SVDQ_OK);
  if (!given_factors && power_iters == 0) {
    EXPECT(svdq_prepare_weights(w.data(), K, N, a.data(), alpha, rank, 64, si.data(), wc.data(), ws.data(),
                                rank ? ld.data() : nullptr, rank ? lu.data() : nullptr) == SVDQ_OK);
  }
}

static void mxfp4_prepare(int K, int N, int rank) {
  auto w = bf16_matrix(static_cast<size_t>(N) * K, 0.02);
  std::vector<float> a(K, 1.5f);
  size_t bytes = 0;
  EXPECT(svdq_prepared_bytes_mxfp4(K, N, rank, &bytes) == SVDQ_OK && bytes > 0);
  std::vector<float> si(K);
  std::vector<uint8_t> wc(static_cast<size_t>(N) * K / 2), ws(static_cast<size_t>(N) * K / 32);
  std::vector<uint16_t> ld(static_cast<size_t>(rank) * K), lu(static_cast<size_t>(N) * rank);
  std::vector<double> sigma(rank > 0 ? rank : 1);
  EXPECT(svdq_prepare_weights_mxfp4(w.data(), K, N, a.data(), 0.5f, rank, nullptr, nullptr, 0, 7u, si.data(),
                                    wc.data(), ws.data(), rank ? ld.data() : nullptr, rank ? lu.data() : nullptr,
                                    sigma.data()) == SVDQ_OK);
}

static void awq_prepare(int K, int N, int Mc, double alpha) {
  auto w = bf16_matrix(static_cast<size_t>(N) * K, 0.02);
  auto x = bf16_matrix(static_cast<size_t>(Mc) * K, 1.0);
  std::vector<float> inv(K);
  std::vector<uint8_t> wc(static_cast<size_t>(N) * K / 2), wz(static_cast<size_t>(N) * K / 64);
  std::vector<uint16_t> ws(static_cast<size_t>(N) * K / 64);
  double al = -2.0;
  EXPECT(svdq_awq_prepare(w.data(), K, N, x.data(), Mc, alpha, 64, inv.data(), wc.data(), ws.data(), wz.data(),
                          &al) == SVDQ_OK);
  EXPECT(al >= 0.0 && al < 1.0);
}

static void fp6_pack(int rows, int K, int layout) {
  size_t bytes = 0;
  EXPECT(svdq_fp6_operand_bytes(rows, K, layout, &bytes) == SVDQ_OK);
  std::vector<uint8_t> codes(static_cast<size_t>(rows) * K / 2);
  for (auto& c : codes) c = static_cast<uint8_t>(uniform() * 256.0);
  std::vector<uint8_t> out(bytes);
  EXPECT(svdq_pack_fp6_operand(codes.data(), rows, K, layout, out.data()) == SVDQ_OK);
}

static void host_argument_checks() {
  size_t b = 0;
  EXPECT(svdq_prepared_bytes(100, 64, 0, 64, &b) != SVDQ_OK);
  EXPECT(svdq_prepared_bytes(64, 64, 0, 64, nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_prepared_bytes(64, 64, 24, 64, &b) != SVDQ_OK);
  EXPECT(svdq_prepared_bytes(-64, 64, 0, 64, &b) != SVDQ_OK);
  EXPECT(svdq_prepared_bytes_mxfp4(96, 64, 0, &b) != SVDQ_OK);
  std::vector<uint16_t> w(64 * 64, 0);
  std::vector<float> a(64, 1.0f), si(64);
  std::vector<uint8_t> wc(64 * 32);
  std::vector<uint16_t> ws(64);
  EXPECT(svdq_prepare_weights(nullptr, 64, 64, a.data(), 0.5f, 0, 64, si.data(), wc.data(), ws.data(), nullptr,
                              nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_prepare_weights(w.data(), 64, 64, a.data(), 0.5f, 16, 64, si.data(), wc.data(), ws.data(), nullptr,
                              nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_prepare_weights(w.data(), 64, 64, a.data(), 0.5f, 80, 64, si.data(), wc.data(), ws.data(), nullptr,
                              nullptr) != SVDQ_OK);
  // a NaN weight is a numeric error, not a crash
  w[5] = 0x7FC0;
  EXPECT(svdq_prepare_weights(w.data(), 64, 64, a.data(), 0.5f, 0, 64, si.data(), wc.data(), ws.data(), nullptr,
                              nullptr) == SVDQ_ERR_NUMERIC);
  EXPECT(svdq_fp6_operand_bytes(1, 100, 0, &b) == SVDQ_ERR_UNSUPPORTED_SHAPE);
  EXPECT(svdq_pack_fp6_operand(nullptr, 1, 64, 0, nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_awq_prepare(nullptr, 64, 32, nullptr, 1, 0.5, 64, nullptr, nullptr, nullptr, nullptr, nullptr) ==
         SVDQ_ERR_INVALID_ARG);
}

// The device entry points: only the argument checks run here.  A call that
// passes them either stops at the device check (no gfx950 visible) or
// reaches a launcher stand-in.
static bool passed_checks(int st) { return st == SVDQ_ERR_UNSUPPORTED_DEVICE || st == 7777; }

static void device_argument_checks() {
  alignas(256) static uint8_t buf[1 << 16];
  void* p = buf;
  float* f = reinterpret_cast<float*>(buf);
  void* odd = buf + 1;
  const int M = 33, K = 128, N = 64, r = 16;
  // kernel 1
  EXPECT(passed_checks(svdq_quant_act_lora_down(p, f, p, M, K, r, 64, SVDQ_ACT_NONE, p, p, f, nullptr)));
  EXPECT(svdq_quant_act_lora_down(p, f, p, M, K, r, 32, SVDQ_ACT_NONE, p, p, f, nullptr) ==
         SVDQ_ERR_UNSUPPORTED_SHAPE);
  EXPECT(svdq_quant_act_lora_down(p, f, p, M, 100, 0, 64, SVDQ_ACT_NONE, p, p, f, nullptr) ==
         SVDQ_ERR_UNSUPPORTED_SHAPE);
  EXPECT(svdq_quant_act_lora_down(p, f, p, -1, K, r, 64, SVDQ_ACT_NONE, p, p, f, nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_quant_act_lora_down(p, f, nullptr, M, K, r, 64, SVDQ_ACT_NONE, p, p, f, nullptr) ==
         SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_quant_act_lora_down(odd, f, p, M, K, r, 64, SVDQ_ACT_NONE, p, p, f, nullptr) ==
         SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_quant_act_lora_down(p, f, p, M, K, r, 64, 9, p, p, f, nullptr) == SVDQ_ERR_INVALID_ARG);
  // kernel 2 and its variants
  EXPECT(passed_checks(svdq_gemm_w4a4_lora_up(p, p, p, p, f, p, nullptr, M, N, K, r, 64, SVDQ_OUT_BF16, p,
                                              nullptr)));
  EXPECT(svdq_gemm_w4a4_lora_up(p, p, p, p, f, p, nullptr, M, 12, K, r, 64, SVDQ_OUT_BF16, p, nullptr) !=
         SVDQ_OK);
  EXPECT(svdq_gemm_w4a4_lora_up(p, p, p, p, f, p, nullptr, M, N, K, r, 64, 5, p, nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_gemm_w4a4_lora_up(p, p, p, p, nullptr, p, nullptr, M, N, K, r, 64, SVDQ_OUT_BF16, p, nullptr) ==
         SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_gemm_w4a4_lora_up(p, p, p, p, f, p, odd, M, N, K, r, 64, SVDQ_OUT_BF16, p, nullptr) ==
         SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_gemm_w4a4_lora_up(p, p, p, p, f, p, nullptr, 1 << 30, N, 1 << 14, 0, 64, SVDQ_OUT_BF16, p,
                                nullptr) == SVDQ_ERR_UNSUPPORTED_SHAPE);
  EXPECT(passed_checks(svdq_gemm_w4a4_lora_up_qkv(p, p, p, p, f, p, nullptr, p, p, f, f, 1e-6f, M, 384, K, r, 64,
                                                  SVDQ_OUT_BF16, p, nullptr)));
  EXPECT(svdq_gemm_w4a4_lora_up_qkv(p, p, p, p, f, p, nullptr, nullptr, p, f, f, 1e-6f, M, 384, K, r, 64,
                                    SVDQ_OUT_BF16, p, nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(passed_checks(svdq_lora_down(p, f, p, M, K, r, 64, SVDQ_ACT_NONE, f, nullptr)));
  EXPECT(svdq_lora_down(p, f, p, M, K, 0, 64, SVDQ_ACT_NONE, f, nullptr) != SVDQ_OK);
  EXPECT(passed_checks(svdq_lora_up_add(f, p, M, N, r, p, nullptr)));
  EXPECT(svdq_lora_up_add(f, p, M, N, r, nullptr, nullptr) == SVDQ_ERR_INVALID_ARG);
  // 6-bit route
  EXPECT(passed_checks(svdq_quant_act_lora_down_fp6(p, f, p, M, K, r, 64, SVDQ_ACT_NONE, p, p, f, nullptr)));
  EXPECT(svdq_quant_act_lora_down_fp6(p, f, p, M, K, r, 64, SVDQ_ACT_NONE, nullptr, p, f, nullptr) ==
         SVDQ_ERR_INVALID_ARG);
  EXPECT(passed_checks(svdq_gemm_w4a4_fp6_lora_up(p, p, p, p, f, p, nullptr, M, N, K, r, 64, SVDQ_OUT_F32, p,
                                                  nullptr)));
  EXPECT(svdq_gemm_w4a4_fp6_lora_up(p, p, p, p, f, p, nullptr, M, N, 96, r, 64, SVDQ_OUT_F32, p, nullptr) !=
         SVDQ_OK);
  EXPECT(passed_checks(svdq_gemm_w4a4_fp6_lora_up_n192(p, p, p, p, f, p, nullptr, M, 384, K, r, 64, SVDQ_OUT_BF16, p,
                                                       nullptr)));
  EXPECT(svdq_gemm_w4a4_fp6_lora_up_n192(p, p, p, p, f, p, nullptr, M, 256, K, r, 64, SVDQ_OUT_BF16, p, nullptr) ==
         SVDQ_ERR_UNSUPPORTED_SHAPE);
  EXPECT(svdq_gemm_w4a4_fp6_lora_up_n192(p, p, p, nullptr, f, p, nullptr, M, 384, K, r, 64, SVDQ_OUT_BF16, p,
                                         nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(passed_checks(svdq_gemm_w4a4_fp6_lora_up_qkv(p, p, p, p, f, p, nullptr, p, p, f, f, 1e-6f, M, 384, K, r,
                                                      64, SVDQ_OUT_BF16, p, nullptr)));
  EXPECT(svdq_gemm_w4a4_fp6_lora_up_qkv(p, p, p, p, f, p, nullptr, p, p, f, nullptr, 1e-6f, M, 384, K, r, 64,
                                        SVDQ_OUT_BF16, p, nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(svdq_gemm_w4a4_fp6_lora_up_qkv(p, p, p, p, f, p, nullptr, p, p, f, f, 1e-6f, M, 256, K, r, 64,
                                        SVDQ_OUT_BF16, p, nullptr) == SVDQ_ERR_UNSUPPORTED_SHAPE);
  // the MLP chain
  size_t ws = 0;
  EXPECT(svdq_mlp_chain_workspace_bytes(M, 512, 32, &ws) == SVDQ_OK && ws == 2u * M * 32 * 4);
  EXPECT(svdq_mlp_chain_workspace_bytes(M, 512, 32, nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(passed_checks(svdq_gemm_w4a4_fp6_mlp_chain(p, p, p, p, f, p, nullptr, M, 512, K, r, 64, f, p, 32, p, p, f,
                                                    p, ws, nullptr)));
  EXPECT(svdq_gemm_w4a4_fp6_mlp_chain(p, p, p, p, f, p, nullptr, M, 512, K, r, 64, f, p, 32, p, p, f, p, ws - 16,
                                      nullptr) == SVDQ_ERR_INVALID_ARG);          // workspace too small
  EXPECT(svdq_gemm_w4a4_fp6_mlp_chain(p, p, p, p, f, p, nullptr, M, 520, K, r, 64, f, p, 32, p, p, f, p, 1 << 20,
                                      nullptr) == SVDQ_ERR_UNSUPPORTED_SHAPE);    // N not a multiple of 64
  EXPECT(svdq_gemm_w4a4_fp6_mlp_chain(p, p, p, p, f, p, nullptr, M, 512, K, r, 64, nullptr, p, 32, p, p, f, p, ws,
                                      nullptr) == SVDQ_ERR_INVALID_ARG);
  EXPECT(passed_checks(svdq_gemm_w4a4_fp6_mlp_chain(p, p, p, p, f, p, nullptr, M, 512, K, r, 64, f, nullptr, 0, p, p,
                                                    nullptr, nullptr, 0, nullptr)));
  EXPECT(passed_checks(svdq_gemm_w4a4_fp6_mlp_chain_noalloc(p, p, p, p, f, p, nullptr, M, 512, K, r, 64, f, p, 32,
                                                            p, p, f, nullptr)));
  EXPECT(svdq_gemm_w4a4_fp6_mlp_chain_noalloc(p, p, p, p, f, p, nullptr, 65536, 12288, K, r, 64, f, p, 16, p, p, f,
                                              nullptr) == SVDQ_ERR_UNSUPPORTED_SHAPE);  // beyond the scratch
  EXPECT(svdq_gemm_w4a4_fp6_mlp_chain_noalloc(p, p, p, p, f, p, nullptr, M, 512, K, r, 64, f, nullptr, 32, p, p, f,
                                              nullptr) == SVDQ_ERR_INVALID_ARG);
  // MXFP4
  EXPECT(passed_checks(svdq_quant_act_lora_down_mxfp4(p, f, p, M, K, r, SVDQ_ACT_NONE, p, p, f, nullptr)));
  EXPECT(svdq_quant_act_lora_down_mxfp4(p, f, p, M, 64, r, SVDQ_ACT_NONE, p, p, f, nullptr) != SVDQ_OK);
  EXPECT(passed_checks(svdq_gemm_mxfp4_lora_up(p, p, p, p, f, p, nullptr, M, N, K, r, SVDQ_OUT_BF16, p, nullptr)));
  // AWQ
  EXPECT(passed_checks(svdq_awq_quant_act(p, f, 4, K, p, f, nullptr)));
  EXPECT(svdq_awq_quant_act(p, f, 17, K, p, f, nullptr) != SVDQ_OK);
  EXPECT(passed_checks(svdq_awq_gemv(p, f, p, p, p, nullptr, 4, 64, K, p, nullptr)));
  EXPECT(svdq_awq_gemv(p, f, p, p, p, nullptr, 4, 48, K, p, nullptr) != SVDQ_OK);
  EXPECT(passed_checks(svdq_awq_linear_row(p, f, p, p, p, nullptr, 64, K, p, nullptr)));
  EXPECT(svdq_awq_linear_row(p, f, p, p, p, nullptr, 64, 8256, p, nullptr) == SVDQ_ERR_UNSUPPORTED_SHAPE);
  EXPECT(svdq_awq_linear_row(p, f, p, p, p, nullptr, 48, K, p, nullptr) == SVDQ_ERR_UNSUPPORTED_SHAPE);
  EXPECT(svdq_awq_linear_row(nullptr, f, p, p, p, nullptr, 64, K, p, nullptr) == SVDQ_ERR_INVALID_ARG);
  // status strings for every code, and an unknown one
  for (int s = -6; s <= 1; ++s) EXPECT(svdq_status_string(s) != nullptr);
  EXPECT(svdq_version() > 0);
  EXPECT(svdq_device_check(-1) == SVDQ_ERR_UNSUPPORTED_DEVICE);
  EXPECT(svdq_device_check(1 << 20) == SVDQ_ERR_UNSUPPORTED_DEVICE);
}

int main() {
  int4_prepare(64, 8, 0, 0.5f, 0, false);
  int4_prepare(128, 24, 16, 0.5f, 0, false);
  int4_prepare(192, 136, 32, 0.25f, 2, false);
  int4_prepare(256, 64, 64, 0.5f, 0, false);
  int4_prepare(320, 40, 16, 0.5f, 0, true);
  mxfp4_prepare(128, 16, 16);
  mxfp4_prepare(256, 40, 0);
  awq_prepare(128, 32, 4, -1.0);
  awq_prepare(192, 64, 3, 0.35);
  for (int layout = 0; layout < 2; ++layout) {
    fp6_pack(1, 64, layout);
    fp6_pack(33, 128, layout);
    fp6_pack(130, 192, layout);
  }
  host_argument_checks();
  device_argument_checks();
  if (g_fail) {
    std::printf("%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("SANITIZE OK (%d launches reached)\n", svdq::g_launches);
  return 0;
}
