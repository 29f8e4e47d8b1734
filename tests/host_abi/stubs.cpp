// Stub kernel launchers and HIP runtime calls for the host-only build of api.cpp (see hip/hip_runtime.h here).
// Each launcher records its name and returns hipSuccess, or the injected error at the chosen call; the runtime
// stubs return their injected errors. Nothing here touches memory behind the pointers it is given.
#include "stubs.h"

#include <string.h>

#include "internal.h"

namespace stub {
std::vector<std::string> calls;
int fail_at = -1;
hipError_t fail_code = hipErrorLaunchFailure;
int syncs = 0;
int sync_fail_at = -1;
hipError_t sync_code = hipErrorIllegalAddress;
hipError_t event_code = hipSuccess;
hipError_t device_code = hipSuccess;
hipError_t symbol_code = hipSuccess;
int device = 0;
int symbol_lookups = 0;
void* workspace_seen = nullptr;

void reset() {
  calls.clear();
  fail_at = -1;
  fail_code = hipErrorLaunchFailure;
  syncs = 0;
  sync_fail_at = -1;
  sync_code = hipErrorIllegalAddress;
  event_code = hipSuccess;
  device_code = hipSuccess;
  symbol_code = hipSuccess;
  device = 0;
  workspace_seen = nullptr;
}

static hipError_t launch(const char* name) {
  const int i = (int)calls.size();
  calls.push_back(name);
  return i == fail_at ? fail_code : hipSuccess;
}
}  // namespace stub

hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return stub::event_code; }
hipError_t hipGetDevice(int* d) {
  *d = stub::device;
  return stub::device_code;
}
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  ++stub::symbol_lookups;
  if (stub::symbol_code != hipSuccess) return stub::symbol_code;
  *ptr = const_cast<void*>(symbol);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) {
  const int i = stub::syncs++;
  return i == stub::sync_fail_at ? stub::sync_code : hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "injected error"; }

namespace sagesla {

hipError_t launch_qk_norm(const Plan&, const uint16_t*, const uint16_t*, hipStream_t) {
  return stub::launch("qk_norm");
}
hipError_t launch_kmean(const Plan&, const uint16_t*, hipStream_t) { return stub::launch("kmean"); }
hipError_t launch_quant(const Plan&, const uint16_t*, const uint16_t*, const uint16_t*, hipStream_t) {
  return stub::launch("quant");
}
hipError_t launch_scores(const Plan&, hipStream_t) { return stub::launch("scores"); }
hipError_t launch_topk(const Plan&, hipStream_t) { return stub::launch("topk"); }
hipError_t launch_linear(const Plan& p, const uint16_t*, const uint16_t*, hipStream_t) {
  stub::workspace_seen = p.keep_mask;
  return stub::launch("linear");
}
hipError_t launch_attn(const Plan& p, const uint16_t*, uint16_t*, hipStream_t) {
  if (!stub::workspace_seen) stub::workspace_seen = p.q_i8;
  return stub::launch("attn");
}
hipError_t launch_w8a8_quant(const uint16_t*, int, int, float, int8_t*, float*, hipStream_t) {
  return stub::launch("w8a8_quant");
}
hipError_t launch_w8a8_gemm(const int8_t*, const float*, const int8_t*, const float*, const uint16_t*, uint16_t*, int,
                            int, int, hipStream_t) {
  return stub::launch("w8a8_gemm");
}
hipError_t launch_backward_sparse(const BwdPlan&, hipStream_t) { return stub::launch("backward_sparse"); }
hipError_t launch_backward_linear(const BwdPlan&, hipStream_t) { return stub::launch("backward_linear"); }
size_t backward_dw_chunks(int N) { return (size_t)(N + 4095) / 4096; }
size_t backward_dw_segments() { return 8; }
size_t backward_norm_chunks(int N) { return (size_t)(N + 1023) / 1024; }
hipError_t launch_norm_backward(const BwdPlan&, const uint16_t*, const uint16_t*, float*, float*, hipStream_t) {
  return stub::launch("norm_backward");
}
hipError_t launch_fill_f32(float*, size_t, float, hipStream_t) { return stub::launch("fill"); }
size_t topk_lds_bytes(int n_kb) { return 1024 + 2 * (size_t)n_kb; }
int mask_row_pad(int n_qb) { return (n_qb + 63) / 64 * 64; }
hipError_t launch_state_sum(const float*, const uint32_t*, float*, int, int, int, int, hipStream_t) {
  return stub::launch("state_sum");
}

}  // namespace sagesla
