// C ABI entry points of the device path: argument validation, the device
// capability check, and dispatch to the kernel launchers.  See include/svdq.h.

#include <hip/hip_runtime.h>
#include <cmath>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "svdq.h"
#include "svdq_internal.h"
#include "svdq_probe.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = supported, 2 = unsupported
std::atomic<int> g_device_ok[kMaxDevices];

int query_device(int dev) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  if (dev < 0 || dev >= count || dev >= kMaxDevices) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  const char* forced = std::getenv("SVDQ_ASSUME_ARCH");
  char arch[256] = {0};
  if (forced) {
    std::strncpy(arch, forced, sizeof(arch) - 1);
  } else {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SVDQ_ERR_HIP;
    std::strncpy(arch, prop.gcnArchName, sizeof(arch) - 1);
  }
  // gcnArchName looks like "gfx950:sramecc+:xnack-"
  return (std::strncmp(arch, "gfx950", 6) == 0 && (arch[6] == 0 || arch[6] == ':'))
             ? SVDQ_OK
             : SVDQ_ERR_UNSUPPORTED_DEVICE;
}

int current_device_check() {
  int dev = -1;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  if (hipGetDevice(&dev) != hipSuccess) return SVDQ_ERR_HIP;
  return svdq_device_check(dev);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The kernels address each operand through a buffer resource whose size
// field is a signed 32-bit byte count.
inline bool fits_buffer(int64_t rows, int64_t bytes_per_row) { return rows * bytes_per_row <= INT32_MAX; }

}  // namespace

namespace svdq {

int device_cu_count() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace svdq

extern "C" const char* svdq_status_string(int status) {
  switch (status) {
    case SVDQ_OK: return "SVDQ_OK";
    case SVDQ_ERR_INVALID_ARG: return "SVDQ_ERR_INVALID_ARG: null pointer, misaligned buffer, or inconsistent size";
    case SVDQ_ERR_UNSUPPORTED_SHAPE: return "SVDQ_ERR_UNSUPPORTED_SHAPE: needs group 64, K % 64 == 0, N % 8 == 0, rank % 16 == 0, rank <= 256";
    case SVDQ_ERR_UNSUPPORTED_DEVICE: return "SVDQ_ERR_UNSUPPORTED_DEVICE: no HIP device, or the device is not gfx950 (MI355X)";
    case SVDQ_ERR_HIP: return "SVDQ_ERR_HIP: a HIP runtime call or kernel launch failed";
    case SVDQ_ERR_NUMERIC: return "SVDQ_ERR_NUMERIC: non-finite input, fp16 scale overflow, or SVD did not converge";
    default: return "SVDQ_ERR_UNKNOWN";
  }
}

extern "C" int svdq_version(void) { return 100; }

extern "C" int svdq_device_check(int hip_device) {
  if (hip_device < 0 || hip_device >= kMaxDevices) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  const int cached = g_device_ok[hip_device].load(std::memory_order_relaxed);
  if (cached == 1) return SVDQ_OK;
  if (cached == 2) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  const int st = query_device(hip_device);
  if (st == SVDQ_OK) g_device_ok[hip_device].store(1, std::memory_order_relaxed);
  else if (st == SVDQ_ERR_UNSUPPORTED_DEVICE) g_device_ok[hip_device].store(2, std::memory_order_relaxed);
  return st;
}

extern "C" int svdq_quant_act_lora_down(const void* x, const float* smooth_inv, const void* lora_down,
                                        int M, int K, int rank, int group, int act, void* x_codes,
                                        void* x_scales, float* lora_act, void* stream) {
  if (M < 0) return SVDQ_ERR_INVALID_ARG;
  if (K <= 0 || rank < 0 || rank > K || group <= 0) return SVDQ_ERR_INVALID_ARG;
  if (group != SVDQ_GROUP || K % group != 0 || rank % 16 != 0 || rank > SVDQ_MAX_RANK || K > 32768)
    return SVDQ_ERR_UNSUPPORTED_SHAPE;
  int st;
  if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
  if (!x || !smooth_inv || !x_codes || !x_scales) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_down || !lora_act)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(smooth_inv) || !aligned16(x_codes) || !aligned16(x_scales) ||
      (rank > 0 && (!aligned16(lora_down) || !aligned16(lora_act))))
    return SVDQ_ERR_INVALID_ARG;
  st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_quant_act_lora_down(x, smooth_inv, lora_down, M, K, rank, act, x_codes, x_scales,
                                          lora_act, stream);
}

extern "C" int svdq_gemm_w4a4_lora_up(const void* x_codes, const void* x_scales, const void* w_codes,
                                      const void* w_scales, const float* lora_act, const void* lora_up,
                                      const void* bias, int M, int N, int K, int rank, int group,
                                      int out_dtype, void* y, void* stream) {
  if (M < 0) return SVDQ_ERR_INVALID_ARG;
  int st = svdq::validate_shape(K, N, rank, group);
  if (st != SVDQ_OK) return st;
  if (out_dtype != SVDQ_OUT_BF16 && out_dtype != SVDQ_OUT_F32) return SVDQ_ERR_INVALID_ARG;
  if (!x_codes || !x_scales || !w_codes || !w_scales || !y) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(y) || (bias && !aligned16(bias)) ||
      (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))))
    return SVDQ_ERR_INVALID_ARG;
  if (!fits_buffer(M, K / 2) || !fits_buffer(N, K / 2)) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_gemm_w4a4_lora_up(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M,
                                        N, K, rank, out_dtype, y, stream);
}

extern "C" int svdq_quant_act_lora_down_fp6(const void* x, const float* smooth_inv, const void* lora_down, int M,
                                            int K, int rank, int group, int act, void* x_fp6, void* x_scales,
                                            float* lora_act, void* stream) {
  if (M < 0 || K <= 0 || rank < 0 || rank > K || group <= 0) return SVDQ_ERR_INVALID_ARG;
  if (group != SVDQ_GROUP || K % group != 0 || rank % 16 != 0 || rank > SVDQ_MAX_RANK || K > 32768)
    return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
  if (!x || !smooth_inv || !x_fp6 || !x_scales) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_down || !lora_act)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(smooth_inv) || !aligned16(x_fp6) || !aligned16(x_scales) ||
      (rank > 0 && (!aligned16(lora_down) || !aligned16(lora_act))))
    return SVDQ_ERR_INVALID_ARG;
  const int64_t RB = (static_cast<int64_t>(M) + 31) / 32;
  if (!fits_buffer(static_cast<int64_t>(K / SVDQ_GROUP) * RB, 1536) || !fits_buffer(M, 2LL * K))
    return SVDQ_ERR_UNSUPPORTED_SHAPE;
  const int st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_quant_act_lora_down_fp6(x, smooth_inv, lora_down, M, K, rank, act, x_fp6, x_scales, lora_act,
                                              stream);
}

extern "C" int svdq_gemm_w4a4_fp6_lora_up(const void* x_fp6, const void* x_scales, const void* w_fp6,
                                          const void* w_scales, const float* lora_act, const void* lora_up,
                                          const void* bias, int M, int N, int K, int rank, int group,
                                          int out_dtype, void* y, void* stream) {
  if (M < 0) return SVDQ_ERR_INVALID_ARG;
  int st = svdq::validate_shape(K, N, rank, group);
  if (st != SVDQ_OK) return st;
  if (out_dtype != SVDQ_OUT_BF16 && out_dtype != SVDQ_OUT_F32) return SVDQ_ERR_INVALID_ARG;
  if (!x_fp6 || !x_scales || !w_fp6 || !w_scales || !y) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x_fp6) || !aligned16(x_scales) || !aligned16(w_fp6) || !aligned16(w_scales) || !aligned16(y) ||
      (bias && !aligned16(bias)) || (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))))
    return SVDQ_ERR_INVALID_ARG;
  const int64_t G = K / SVDQ_GROUP;
  const int64_t RBa = (static_cast<int64_t>(M) + 31) / 32, RBb = 4 * ((static_cast<int64_t>(N) + 127) / 128);
  // every operand and the output are addressed through buffer descriptors
  // with 32-bit offsets
  if (!fits_buffer(G * RBa, 1536) || !fits_buffer(G * RBb, 1536) || !fits_buffer(G, 64LL * RBa) ||
      !fits_buffer(G, 2LL * N) || !fits_buffer(M, 4LL * rank) ||
      !fits_buffer(M, static_cast<int64_t>(N) * (out_dtype == SVDQ_OUT_F32 ? 4 : 2)))
    return SVDQ_ERR_UNSUPPORTED_SHAPE;
  st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_gemm_w4a4_fp6(x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias, M, N, K, rank,
                                    out_dtype, y, stream);
}

extern "C" int svdq_gemm_w4a4_fp6_lora_up_n192(const void* x_fp6, const void* x_scales, const void* w_fp6,
                                               const void* w_scales, const float* lora_act, const void* lora_up,
                                               const void* bias, int M, int N, int K, int rank, int group,
                                               int out_dtype, void* y, void* stream) {
  if (M < 0) return SVDQ_ERR_INVALID_ARG;
  int st = svdq::validate_shape(K, N, rank, group);
  if (st != SVDQ_OK) return st;
  if (N % 192 != 0) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (out_dtype != SVDQ_OUT_BF16 && out_dtype != SVDQ_OUT_F32) return SVDQ_ERR_INVALID_ARG;
  if (!x_fp6 || !x_scales || !w_fp6 || !w_scales || !y) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x_fp6) || !aligned16(x_scales) || !aligned16(w_fp6) || !aligned16(w_scales) || !aligned16(y) ||
      (bias && !aligned16(bias)) || (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))))
    return SVDQ_ERR_INVALID_ARG;
  const int64_t G = K / SVDQ_GROUP;
  const int64_t RBa = (static_cast<int64_t>(M) + 31) / 32, RBw = N / 32;
  if (!fits_buffer(G * RBa, 1536) || !fits_buffer(G * RBw, 1536) || !fits_buffer(G, 64LL * RBa) ||
      !fits_buffer(G, 2LL * N) || !fits_buffer(M, 4LL * rank) ||
      !fits_buffer(M, static_cast<int64_t>(N) * (out_dtype == SVDQ_OUT_F32 ? 4 : 2)))
    return SVDQ_ERR_UNSUPPORTED_SHAPE;
  st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_gemm_w4a4_fp6_n192(x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias, M, N, K, rank,
                                         out_dtype, y, stream);
}

extern "C" int svdq_fp6_n192_preferred(int M, int N) { return svdq::fp6_n192_preferred(M, N); }

extern "C" int svdq_int4_route(int M, int N) { return svdq::fp6_route(M, N); }

extern "C" int svdq_gemm_w4a4_fp6_lora_up_qkv(const void* x_fp6, const void* x_scales, const void* w_fp6,
                                              const void* w_scales, const float* lora_act, const void* lora_up,
                                              const void* bias, const void* norm_q, const void* norm_k,
                                              const float* rope_cos, const float* rope_sin, float eps, int M, int N,
                                              int K, int rank, int group, int out_dtype, void* y, void* stream) {
  if (M < 0) return SVDQ_ERR_INVALID_ARG;
  int st = svdq::validate_shape(K, N, rank, group);
  if (st != SVDQ_OK) return st;
  if (N % (3 * SVDQ_QKV_HEAD_DIM) != 0) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (out_dtype != SVDQ_OUT_BF16 && out_dtype != SVDQ_OUT_F32) return SVDQ_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return SVDQ_ERR_INVALID_ARG;
  if (!x_fp6 || !x_scales || !w_fp6 || !w_scales || !y || !norm_q || !norm_k) return SVDQ_ERR_INVALID_ARG;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x_fp6) || !aligned16(x_scales) || !aligned16(w_fp6) || !aligned16(w_scales) || !aligned16(y) ||
      (bias && !aligned16(bias)) || !aligned16(norm_q) || !aligned16(norm_k) ||
      (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) ||
      (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))))
    return SVDQ_ERR_INVALID_ARG;
  const int64_t G = K / SVDQ_GROUP;
  const int64_t RBa = (static_cast<int64_t>(M) + 31) / 32, RBb = 4 * ((static_cast<int64_t>(N) + 127) / 128);
  if (!fits_buffer(G * RBa, 1536) || !fits_buffer(G * RBb, 1536) || !fits_buffer(G, 64LL * RBa) ||
      !fits_buffer(G, 2LL * N) || !fits_buffer(M, 4LL * rank) ||
      !fits_buffer(M, static_cast<int64_t>(N) * (out_dtype == SVDQ_OUT_F32 ? 4 : 2)) ||
      (rope_cos && !fits_buffer(M, 64 * sizeof(float))))
    return SVDQ_ERR_UNSUPPORTED_SHAPE;
  st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_gemm_w4a4_fp6_qkv(x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias, norm_q, norm_k,
                                        rope_cos, rope_sin, eps, M, N, K, rank, out_dtype, y, stream);
}

namespace {
// Argument checks of the MLP chain (both entry points); the workspace is
// checked by the caller.
int check_chain(const void* x_fp6, const void* x_scales, const void* w_fp6, const void* w_scales,
                const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K, int rank,
                int group, const float* smooth_inv_dn, const void* lora_down_dn, int rank_dn, const void* x_fp6_dn,
                const void* x_scales_dn, const float* lora_act_dn) {
  if (M < 0 || rank_dn < 0) return SVDQ_ERR_INVALID_ARG;
  const int st = svdq::validate_shape(K, N, rank, group);
  if (st != SVDQ_OK) return st;
  if (N % SVDQ_GROUP != 0 || rank_dn % 16 != 0 || rank_dn > SVDQ_MAX_RANK || rank_dn > N)
    return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (!x_fp6 || !x_scales || !w_fp6 || !w_scales || !smooth_inv_dn || !x_fp6_dn || !x_scales_dn)
    return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (rank_dn > 0 && (!lora_down_dn || !lora_act_dn)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x_fp6) || !aligned16(x_scales) || !aligned16(w_fp6) || !aligned16(w_scales) ||
      !aligned16(smooth_inv_dn) || !aligned16(x_fp6_dn) || !aligned16(x_scales_dn) || (bias && !aligned16(bias)) ||
      (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))) ||
      (rank_dn > 0 && (!aligned16(lora_down_dn) || !aligned16(lora_act_dn))))
    return SVDQ_ERR_INVALID_ARG;
  const int64_t G = K / SVDQ_GROUP, Gd = N / SVDQ_GROUP;
  const int64_t RBa = (static_cast<int64_t>(M) + 31) / 32, RBb = 4 * ((static_cast<int64_t>(N) + 127) / 128);
  if (!fits_buffer(G * RBa, 1536) || !fits_buffer(G * RBb, 1536) || !fits_buffer(G, 64LL * RBa) ||
      !fits_buffer(G, 2LL * N) || !fits_buffer(Gd * RBa, 1536) || !fits_buffer(M, 4LL * rank))
    return SVDQ_ERR_UNSUPPORTED_SHAPE;
  return SVDQ_OK;
}
}  // namespace

extern "C" int svdq_mlp_chain_workspace_bytes(int M, int N, int rank_dn, size_t* bytes_out) {
  if (M < 0 || N < 0 || rank_dn < 0 || !bytes_out) return SVDQ_ERR_INVALID_ARG;
  *bytes_out = static_cast<size_t>((N + 255) / 256) * static_cast<size_t>(M) * static_cast<size_t>(rank_dn) * 4u;
  return SVDQ_OK;
}

extern "C" int svdq_gemm_w4a4_fp6_mlp_chain(const void* x_fp6, const void* x_scales, const void* w_fp6,
                                            const void* w_scales, const float* lora_act, const void* lora_up,
                                            const void* bias, int M, int N, int K, int rank, int group,
                                            const float* smooth_inv_dn, const void* lora_down_dn, int rank_dn,
                                            void* x_fp6_dn, void* x_scales_dn, float* lora_act_dn, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  int st = check_chain(x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias, M, N, K, rank, group,
                       smooth_inv_dn, lora_down_dn, rank_dn, x_fp6_dn, x_scales_dn, lora_act_dn);
  if (st != SVDQ_OK) return st;
  size_t need = 0;
  svdq_mlp_chain_workspace_bytes(M, N, rank_dn, &need);
  if (rank_dn > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need)) return SVDQ_ERR_INVALID_ARG;
  st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_mlp_chain_fp6(x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias, M, N, K, rank,
                                    smooth_inv_dn, lora_down_dn, rank_dn, x_fp6_dn, x_scales_dn, lora_act_dn,
                                    static_cast<float*>(workspace), stream);
}

extern "C" int svdq_gemm_w4a4_fp6_mlp_chain_noalloc(const void* x_fp6, const void* x_scales, const void* w_fp6,
                                                    const void* w_scales, const float* lora_act, const void* lora_up,
                                                    const void* bias, int M, int N, int K, int rank, int group,
                                                    const float* smooth_inv_dn, const void* lora_down_dn, int rank_dn,
                                                    void* x_fp6_dn, void* x_scales_dn, float* lora_act_dn,
                                                    void* stream) {
  int st = check_chain(x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias, M, N, K, rank, group,
                       smooth_inv_dn, lora_down_dn, rank_dn, x_fp6_dn, x_scales_dn, lora_act_dn);
  if (st != SVDQ_OK) return st;
  size_t need = 0;
  svdq_mlp_chain_workspace_bytes(M, N, rank_dn, &need);
  if (need > svdq::chain_scratch_bytes()) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  void* ws = nullptr;
  if (rank_dn > 0) {
    st = svdq::chain_scratch(&ws);
    if (st != SVDQ_OK) return st;
  }
  return svdq::launch_mlp_chain_fp6(x_fp6, x_scales, w_fp6, w_scales, lora_act, lora_up, bias, M, N, K, rank,
                                    smooth_inv_dn, lora_down_dn, rank_dn, x_fp6_dn, x_scales_dn, lora_act_dn,
                                    static_cast<float*>(ws), stream);
}

extern "C" int svdq_lora_down(const void* x, const float* smooth_inv, const void* lora_down, int M, int K,
                              int rank, int group, int act, float* lora_act, void* stream) {
  if (M < 0 || K <= 0 || rank <= 0 || rank > K || group <= 0) return SVDQ_ERR_INVALID_ARG;
  if (group != SVDQ_GROUP || K % group != 0 || rank % 16 != 0 || rank > SVDQ_MAX_RANK || K > 32768)
    return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
  if (!x || !smooth_inv || !lora_down || !lora_act) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(smooth_inv) || !aligned16(lora_down) || !aligned16(lora_act))
    return SVDQ_ERR_INVALID_ARG;
  const int st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_lora_down(x, smooth_inv, lora_down, M, K, rank, act, lora_act, stream);
}

extern "C" int svdq_lora_up_add(const float* lora_act, const void* lora_up, int M, int N, int rank, void* y,
                                void* stream) {
  if (M < 0 || N <= 0 || rank <= 0 || rank > N) return SVDQ_ERR_INVALID_ARG;
  if (N % 8 != 0 || rank % 16 != 0 || rank > SVDQ_MAX_RANK) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (!lora_act || !lora_up || !y) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(lora_act) || !aligned16(lora_up) || !aligned16(y)) return SVDQ_ERR_INVALID_ARG;
  const int st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_lora_up_add(lora_act, lora_up, M, N, rank, y, stream);
}

extern "C" int svdq_quant_act_lora_down_mxfp4(const void* x, const float* smooth_inv, const void* lora_down,
                                              int M, int K, int rank, int act, void* x_codes, void* x_scales,
                                              float* lora_act, void* stream) {
  if (M < 0 || K <= 0 || rank < 0 || rank > K) return SVDQ_ERR_INVALID_ARG;
  if (K % 128 != 0 || rank % 16 != 0 || rank > SVDQ_MAX_RANK || K > 32768) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
  if (!x || !smooth_inv || !x_codes || !x_scales) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_down || !lora_act)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(smooth_inv) || !aligned16(x_codes) || !aligned16(x_scales) ||
      (rank > 0 && (!aligned16(lora_down) || !aligned16(lora_act))))
    return SVDQ_ERR_INVALID_ARG;
  const int st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_quant_act_lora_down_mxfp4(x, smooth_inv, lora_down, M, K, rank, act, x_codes, x_scales,
                                                lora_act, stream);
}

extern "C" int svdq_gemm_mxfp4_lora_up(const void* x_codes, const void* x_scales, const void* w_codes,
                                       const void* w_scales, const float* lora_act, const void* lora_up,
                                       const void* bias, int M, int N, int K, int rank, int out_dtype,
                                       void* y, void* stream) {
  if (M < 0) return SVDQ_ERR_INVALID_ARG;
  int st = svdq::validate_shape_mx(K, N, rank);
  if (st != SVDQ_OK) return st;
  if (out_dtype != SVDQ_OUT_BF16 && out_dtype != SVDQ_OUT_F32) return SVDQ_ERR_INVALID_ARG;
  if (!x_codes || !x_scales || !w_codes || !w_scales || !y) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(y) || (bias && !aligned16(bias)) ||
      (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))))
    return SVDQ_ERR_INVALID_ARG;
  if (!fits_buffer(M, K / 2) || !fits_buffer(N, K / 2)) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_gemm_mxfp4_lora_up(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N,
                                         K, rank, out_dtype, y, stream);
}

extern "C" int svdq_gemm_w4a4_lora_up_qkv(const void* x_codes, const void* x_scales, const void* w_codes,
                                          const void* w_scales, const float* lora_act, const void* lora_up,
                                          const void* bias, const void* norm_q, const void* norm_k,
                                          const float* rope_cos, const float* rope_sin, float eps, int M, int N,
                                          int K, int rank, int group, int out_dtype, void* y, void* stream) {
  if (M < 0) return SVDQ_ERR_INVALID_ARG;
  int st = svdq::validate_shape(K, N, rank, group);
  if (st != SVDQ_OK) return st;
  if (N % (3 * SVDQ_QKV_HEAD_DIM) != 0) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (out_dtype != SVDQ_OUT_BF16 && out_dtype != SVDQ_OUT_F32) return SVDQ_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return SVDQ_ERR_INVALID_ARG;
  if (!x_codes || !x_scales || !w_codes || !w_scales || !y || !norm_q || !norm_k) return SVDQ_ERR_INVALID_ARG;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(y) || (bias && !aligned16(bias)) || !aligned16(norm_q) || !aligned16(norm_k) ||
      (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) ||
      (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))))
    return SVDQ_ERR_INVALID_ARG;
  if (!fits_buffer(M, K / 2) || !fits_buffer(N, K / 2)) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (rope_cos && !fits_buffer(M, 64 * sizeof(float))) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_gemm_w4a4_lora_up_qkv(x_codes, x_scales, w_codes, w_scales, lora_act, lora_up, bias, norm_q,
                                            norm_k, rope_cos, rope_sin, eps, M, N, K, rank, out_dtype, y, stream);
}

extern "C" int svdq_awq_quant_act(const void* x, const float* inv_scale, int M, int K, void* x_hat, float* xsum,
                                  void* stream) {
  if (M < 0 || K <= 0) return SVDQ_ERR_INVALID_ARG;
  if (K % SVDQ_GROUP != 0 || M > SVDQ_AWQ_MAX_ROWS) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (!x || !inv_scale || !x_hat || !xsum) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(inv_scale) || !aligned16(x_hat) || !aligned16(xsum)) return SVDQ_ERR_INVALID_ARG;
  const int st = current_device_check();
  if (st != SVDQ_OK) return st;
  return svdq::launch_awq_quant_act(x, inv_scale, M, K, x_hat, xsum, stream);
}

extern "C" int svdq_awq_gemv(const void* x_hat, const float* xsum, const void* w_codes, const void* w_scales,
                             const void* w_zeros, const void* bias, int M, int N, int K, void* y, void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return SVDQ_ERR_INVALID_ARG;
  if (K % SVDQ_GROUP != 0 || N % 32 != 0 || M > SVDQ_AWQ_MAX_ROWS) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (!x_hat || !xsum || !w_codes || !w_scales || !w_zeros || !y) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x_hat) || !aligned16(xsum) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(w_zeros) ||
      !aligned16(y) || (bias && !aligned16(bias)))
    return SVDQ_ERR_INVALID_ARG;
  if (!fits_buffer(N, K / 2) || !fits_buffer(M, 2LL * K)) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  const int st = current_device_check();
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  return svdq::launch_awq_gemv(x_hat, xsum, w_codes, w_scales, w_zeros, bias, M, N, K, y, stream);
}

extern "C" int svdq_awq_linear_row(const void* x, const float* inv_scale, const void* w_codes, const void* w_scales,
                                   const void* w_zeros, const void* bias, int N, int K, void* y, void* stream) {
  if (N <= 0 || K <= 0) return SVDQ_ERR_INVALID_ARG;
  if (K % SVDQ_GROUP != 0 || N % 32 != 0 || K > SVDQ_AWQ_ROW_MAX_K) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (!x || !inv_scale || !w_codes || !w_scales || !w_zeros || !y) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(inv_scale) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(w_zeros) ||
      !aligned16(y) || (bias && !aligned16(bias)))
    return SVDQ_ERR_INVALID_ARG;
  if (!fits_buffer(N, K / 2)) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  const int st = current_device_check();
  if (st != SVDQ_OK) return st;
  return svdq::launch_awq_linear_row(x, inv_scale, w_codes, w_scales, w_zeros, bias, N, K, y, stream);
}

extern "C" int svdq_probe_mfma(int kind, int blocks, int iters, void* sink, void* stream) {
  if (kind < SVDQ_PROBE_MFMA_I8 || kind > SVDQ_PROBE_FP6_DEQUANT) return SVDQ_ERR_INVALID_ARG;
  if (blocks < 1 || iters < 1 || !sink || !aligned16(sink)) return SVDQ_ERR_INVALID_ARG;
  const int st = current_device_check();
  if (st != SVDQ_OK) return st;
  return svdq::launch_probe_mfma(kind, blocks, iters, sink, stream);
}

extern "C" double svdq_probe_mfma_ops(int kind, int blocks, int iters) {
  if (kind < SVDQ_PROBE_MFMA_I8 || kind > SVDQ_PROBE_FP6_DEQUANT || blocks < 1 || iters < 1) return 0.0;
  return svdq::probe_mfma_ops(kind, blocks, iters);
}
