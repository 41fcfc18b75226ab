// Launcher stand-ins for the host-only sanitizer build of the C ABI: every
// argument check in svdq_abi.hip runs as in the library, and a call that
// passes them reaches one of these, which records that it was reached and
// returns a marker status instead of launching a kernel.
#include <cstddef>

#include "svdq_internal.h"

namespace svdq {
int g_launches = 0;
constexpr int kReached = 7777;

int launch_quant_act_lora_down(const void*, const float*, const void*, int, int, int, int, void*, void*, float*,
                               void*) { ++g_launches; return kReached; }
int launch_lora_down(const void*, const float*, const void*, int, int, int, int, float*, void*) {
  ++g_launches; return kReached; }
int launch_lora_up_add(const float*, const void*, int, int, int, void*, void*) { ++g_launches; return kReached; }
int launch_gemm_w4a4_lora_up(const void*, const void*, const void*, const void*, const float*, const void*,
                             const void*, int, int, int, int, int, void*, void*) { ++g_launches; return kReached; }
int launch_gemm_w4a4_lora_up_qkv(const void*, const void*, const void*, const void*, const float*, const void*,
                                 const void*, const void*, const void*, const float*, const float*, float, int, int,
                                 int, int, int, void*, void*) { ++g_launches; return kReached; }
int launch_quant_act_lora_down_mxfp4(const void*, const float*, const void*, int, int, int, int, void*, void*,
                                     float*, void*) { ++g_launches; return kReached; }
int launch_gemm_mxfp4_lora_up(const void*, const void*, const void*, const void*, const float*, const void*,
                              const void*, int, int, int, int, int, void*, void*) { ++g_launches; return kReached; }
int launch_awq_quant_act(const void*, const float*, int, int, void*, float*, void*) { ++g_launches; return kReached; }
int launch_awq_gemv(const void*, const float*, const void*, const void*, const void*, const void*, int, int, int,
                    void*, void*) { ++g_launches; return kReached; }
int launch_awq_linear_row(const void*, const float*, const void*, const void*, const void*, const void*, int, int,
                          void*, void*) { ++g_launches; return kReached; }
int launch_quant_act_lora_down_fp6(const void*, const float*, const void*, int, int, int, int, void*, void*, float*,
                                   void*) { ++g_launches; return kReached; }
int launch_gemm_w4a4_fp6(const void*, const void*, const void*, const void*, const float*, const void*, const void*,
                         int, int, int, int, int, void*, void*) { ++g_launches; return kReached; }
int launch_gemm_w4a4_fp6_n192(const void*, const void*, const void*, const void*, const float*, const void*,
                              const void*, int, int, int, int, int, void*, void*) { ++g_launches; return kReached; }
int fp6_n192_preferred(int, int) { return 0; }
int fp6_route(int, int) { return 0; }
int launch_gemm_w4a4_fp6_qkv(const void*, const void*, const void*, const void*, const float*, const void*,
                             const void*, const void*, const void*, const float*, const float*, float, int, int, int,
                             int, int, void*, void*) { ++g_launches; return kReached; }
int launch_mlp_chain_fp6(const void*, const void*, const void*, const void*, const float*, const void*, const void*,
                         int, int, int, int, const float*, const void*, int, void*, void*, float*, float*, void*) {
  ++g_launches; return kReached; }
int launch_probe_mfma(int, int, int, void*, void*) { ++g_launches; return kReached; }
size_t chain_scratch_bytes() { return size_t{32} << 20; }
int chain_scratch(void** ptr) {
  static unsigned char stand_in[16];
  *ptr = stand_in;
  return 0;
}
double probe_mfma_ops(int, int, int) { return 0.0; }
}  // namespace svdq
