// Host-only checks of the C ABI (api.cpp built against the stub launchers and HIP runtime of stubs.cpp): every
// validation code of every entry point, the launch order of each stage, SAGESLA_E_HIP and sagesla_last_hip_error for
// a failure injected at every launch, the allocation-free entry point's scratch lookup, and (argument "debug", run
// with SAGESLA_DEBUG=1) the synchronizing debug mode. Exits non-zero on the first failed check.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <thread>
#include <vector>

#include "sagesla.h"
#include "stubs.h"
#include "w8a8.h"

static int g_checks = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    ++g_checks;                                                            \
    if (!(cond)) {                                                         \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      exit(1);                                                             \
    }                                                                      \
  } while (0)

typedef std::vector<std::string> Seq;

// fake device addresses: never dereferenced by the host code or the stubs
static void* addr(uintptr_t a) { return (void*)a; }
static void* const kQ = addr(0x10000000), *const kK = addr(0x20000000), *const kV = addr(0x30000000);
static void* const kOut = addr(0x40000000), *const kW = addr(0x50000000), *const kWs = addr(0x60000000);

static sagesla_params base(int N = 1000, int topk = 4) {
  sagesla_params p;
  memset(&p, 0, sizeof p);
  p.B = 1;
  p.H = 2;
  p.N = N;
  p.D = 128;
  p.blk_q = 128;
  p.blk_k = 64;
  p.topk = topk;
  p.flags = SAGESLA_LINEAR | SAGESLA_SMOOTH_K;
  p.w_proj = kW;
  p.workspace = kWs;
  p.workspace_bytes = sagesla_workspace_bytes(&p);
  return p;
}

static sagesla_status fwd(const sagesla_params& p) { return sagesla_forward(kQ, kK, kV, kOut, &p, nullptr); }

// a run must succeed with exactly this launch order; then a failure injected at each launch must stop the run
// there with SAGESLA_E_HIP and the injected code
template <class F>
static void check_sequence(F run, const Seq& expect, bool debug) {
  stub::reset();
  CHECK(run() == SAGESLA_OK);
  CHECK(stub::calls == expect);
  CHECK(stub::syncs == (debug ? (int)expect.size() : 0));
  for (int i = 0; i < (int)expect.size(); ++i) {
    stub::reset();
    stub::fail_at = i;
    stub::fail_code = (hipError_t)(700 + i);
    CHECK(run() == SAGESLA_E_HIP);
    CHECK(sagesla_last_hip_error() == 700 + i);
    CHECK((int)stub::calls.size() == i + 1);
  }
  if (debug) {  // a fault seen by the synchronization after launch i
    for (int i = 0; i < (int)expect.size(); ++i) {
      stub::reset();
      stub::sync_fail_at = i;
      stub::sync_code = (hipError_t)(800 + i);
      CHECK(run() == SAGESLA_E_HIP);
      CHECK(sagesla_last_hip_error() == 800 + i);
      CHECK((int)stub::calls.size() == i + 1);
    }
  }
  stub::reset();
}

static void status_strings() {
  const char* s[7];
  for (int i = 0; i < 7; ++i) {
    s[i] = sagesla_status_str((sagesla_status)i);
    CHECK(s[i] && s[i][0]);
    for (int j = 0; j < i; ++j) CHECK(strcmp(s[i], s[j]) != 0);
  }
  CHECK(strcmp(sagesla_status_str((sagesla_status)99), "unknown status") == 0);
}

static void validation() {
  CHECK(sagesla_validate(nullptr) == SAGESLA_E_NULL);
  CHECK(sagesla_workspace_bytes(nullptr) == 0);
  sagesla_params p = base();
  CHECK(sagesla_validate(&p) == SAGESLA_OK);
  struct Case {
    void (*set)(sagesla_params&);
    sagesla_status want;
  };
  const Case cases[] = {
      {[](sagesla_params& q) { q.D = 64; }, SAGESLA_E_UNSUPPORTED},
      {[](sagesla_params& q) { q.blk_k = 32; }, SAGESLA_E_UNSUPPORTED},
      {[](sagesla_params& q) { q.blk_q = 96; }, SAGESLA_E_UNSUPPORTED},
      {[](sagesla_params& q) { q.flags |= 0x100u; }, SAGESLA_E_UNSUPPORTED},
      {[](sagesla_params& q) { q.B = 0; }, SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.H = -1; }, SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.N = 0; }, SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.B = 256; q.H = 256; }, SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.N = (1 << 24) + 1; }, SAGESLA_E_UNSUPPORTED},
      {[](sagesla_params& q) { q.N = 20481 * 64; }, SAGESLA_E_UNSUPPORTED},
      {[](sagesla_params& q) { q.topk = -1; }, SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.topk = 17; }, SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.sm_scale = NAN; }, SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.sm_scale = -1.f; }, SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.sm_scale = INFINITY; }, SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.w_proj = nullptr; }, SAGESLA_E_NULL},
      {[](sagesla_params& q) { q.flags |= SAGESLA_QK_RMSNORM; }, SAGESLA_E_NULL},
      {[](sagesla_params& q) { q.flags |= SAGESLA_QK_RMSNORM; q.q_norm_w = kW; q.k_norm_w = kW; q.norm_eps = NAN; },
       SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.flags |= SAGESLA_QK_RMSNORM; q.q_norm_w = kW; q.k_norm_w = kW; q.norm_eps = -1e-6f; },
       SAGESLA_E_SHAPE},
      {[](sagesla_params& q) { q.w_proj = addr(0x50000008); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.q_i8 = (int8_t*)addr(0x70000004); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.k_i8 = (int8_t*)addr(0x70000001); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.q_scale = (float*)addr(0x70000004); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.k_scale = (float*)addr(0x70000004); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.k_mean = (float*)addr(0x70000004); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.q_pool = (double*)addr(0x70000008); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.k_pool = (double*)addr(0x70000008); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.block_idx = (int32_t*)addr(0x70000004); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.o_lin = (float*)addr(0x70000004); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.scores = (double*)addr(0x70000008); }, SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.flags |= SAGESLA_QK_RMSNORM; q.q_norm_w = addr(0x50000002); q.k_norm_w = kW; },
       SAGESLA_E_ALIGN},
      {[](sagesla_params& q) { q.flags |= SAGESLA_QK_RMSNORM; q.q_norm_w = kW; q.k_norm_w = kW;
                               q.q_hat = addr(0x70000002); }, SAGESLA_E_ALIGN},
  };
  for (const Case& c : cases) {
    sagesla_params q = base();
    c.set(q);
    CHECK(sagesla_validate(&q) == c.want);
    stub::reset();
    CHECK(fwd(q) == c.want);  // every entry point validates first and launches nothing on a failure
    CHECK(sagesla_quantize(kQ, kK, &q, nullptr) == c.want);
    CHECK(sagesla_select(&q, nullptr) == c.want);
    CHECK(stub::calls.empty());
    if (c.want != SAGESLA_E_NULL && c.want != SAGESLA_E_ALIGN) CHECK(sagesla_workspace_bytes(&q) == 0);
  }
  // valid corner values
  p = base(1000, 0);
  CHECK(sagesla_validate(&p) == SAGESLA_OK);
  p = base(1000, 16);  // topk == n_kb
  CHECK(sagesla_validate(&p) == SAGESLA_OK);
  p = base(20480 * 64, 2048);  // the largest key-block count
  CHECK(sagesla_validate(&p) == SAGESLA_OK && sagesla_workspace_bytes(&p) > 0);
  p = base();
  p.B = 255;
  p.H = 257;  // B * H = 65535
  CHECK(sagesla_validate(&p) == SAGESLA_OK && sagesla_workspace_bytes(&p) > 0);
  p = base(1, 1);  // one token
  CHECK(sagesla_validate(&p) == SAGESLA_OK);
  p = base();
  p.sm_scale = 0.f;
  CHECK(sagesla_validate(&p) == SAGESLA_OK);
  p.flags &= ~SAGESLA_LINEAR;
  p.w_proj = nullptr;
  CHECK(sagesla_validate(&p) == SAGESLA_OK);
}

static void workspace_sizes() {
  sagesla_params a = base(1000), b = base(4000);
  CHECK(a.workspace_bytes > 0 && b.workspace_bytes > a.workspace_bytes);
  sagesla_params nolin = base(1000);
  nolin.flags &= ~SAGESLA_LINEAR;
  CHECK(sagesla_workspace_bytes(&nolin) < a.workspace_bytes);
  sagesla_params all = base(1000, 16);  // every block selected: no linear branch state
  sagesla_params all_nolin = all;
  all_nolin.flags &= ~SAGESLA_LINEAR;
  CHECK(sagesla_workspace_bytes(&all) == sagesla_workspace_bytes(&all_nolin));
  CHECK(a.workspace_bytes % 256 == 0);
  CHECK(sagesla_backward_workspace_bytes(&a) > 0);
  sagesla_params bad = base();
  bad.D = 64;
  CHECK(sagesla_backward_workspace_bytes(&bad) == 0);
}

static void forward(bool debug) {
  sagesla_params p = base();
  // pointers passed beside the parameter block
  CHECK(sagesla_forward(nullptr, kK, kV, kOut, &p, nullptr) == SAGESLA_E_NULL);
  CHECK(sagesla_forward(kQ, nullptr, kV, kOut, &p, nullptr) == SAGESLA_E_NULL);
  CHECK(sagesla_forward(kQ, kK, nullptr, kOut, &p, nullptr) == SAGESLA_E_NULL);
  CHECK(sagesla_forward(kQ, kK, kV, nullptr, &p, nullptr) == SAGESLA_E_NULL);
  CHECK(sagesla_forward(addr(0x10000002), kK, kV, kOut, &p, nullptr) == SAGESLA_E_ALIGN);
  CHECK(sagesla_forward(kQ, kK, kV, addr(0x40000008), &p, nullptr) == SAGESLA_E_ALIGN);
  CHECK(sagesla_forward(kQ, kK, kV, kOut, nullptr, nullptr) == SAGESLA_E_NULL);
  sagesla_params g = p;
  g.flags |= SAGESLA_USE_GIVEN_MASK;
  CHECK(fwd(g) == SAGESLA_E_NULL);
  // workspace
  sagesla_params w = p;
  w.workspace = nullptr;
  CHECK(fwd(w) == SAGESLA_E_WORKSPACE);
  w = p;
  w.workspace_bytes -= 1;
  CHECK(fwd(w) == SAGESLA_E_WORKSPACE);
  w = p;
  w.workspace = addr(0x60000080);
  CHECK(fwd(w) == SAGESLA_E_ALIGN);
  CHECK(stub::calls.empty());

  auto run = [](const sagesla_params& q) { return [q] { return fwd(q); }; };
  check_sequence(run(p), {"kmean", "quant", "scores", "topk", "linear", "attn"}, debug);
  sagesla_params n = p;
  n.flags |= SAGESLA_QK_RMSNORM;
  n.q_norm_w = n.k_norm_w = kW;
  n.workspace_bytes = sagesla_workspace_bytes(&n);
  check_sequence(run(n), {"qk_norm", "kmean", "quant", "scores", "topk", "linear", "attn"}, debug);
  g.block_idx = (int32_t*)addr(0x70000000);
  check_sequence(run(g), {"kmean", "quant", "linear", "attn"}, debug);
  sagesla_params all = base(1000, 16);  // every block selected: no scores, no linear branch
  check_sequence(run(all), {"kmean", "quant", "topk", "attn"}, debug);
  all.o_lin = (float*)addr(0x70000000);  // its export is then filled with zeros
  check_sequence(run(all), {"kmean", "quant", "topk", "fill", "attn"}, debug);
  sagesla_params none = base(1000, 0);
  check_sequence(run(none), {"kmean", "quant", "linear", "attn"}, debug);
  // timing events: a failing record is reported like a failing launch
  void* evs[2 * SAGESLA_NUM_STAGES];
  for (int i = 0; i < 2 * SAGESLA_NUM_STAGES; ++i) evs[i] = addr(0x80000000 + 16 * i);
  sagesla_params e = p;
  e.events = evs;
  stub::reset();
  CHECK(fwd(e) == SAGESLA_OK);
  stub::event_code = hipErrorInvalidValue;
  CHECK(fwd(e) == SAGESLA_E_HIP);
  CHECK(sagesla_last_hip_error() == hipErrorInvalidValue);
  stub::reset();
}

static void quantize_select(bool debug) {
  sagesla_params p = base();
  CHECK(sagesla_quantize(nullptr, kK, &p, nullptr) == SAGESLA_E_NULL);
  CHECK(sagesla_quantize(kQ, addr(0x20000004), &p, nullptr) == SAGESLA_E_ALIGN);
  sagesla_params w = p;
  w.workspace_bytes = 16;
  CHECK(sagesla_quantize(kQ, kK, &w, nullptr) == SAGESLA_E_WORKSPACE);
  CHECK(sagesla_select(&w, nullptr) == SAGESLA_E_WORKSPACE);
  check_sequence([p] { return sagesla_quantize(kQ, kK, &p, nullptr); }, {"kmean", "quant"}, debug);
  check_sequence([p] { return sagesla_select(&p, nullptr); }, {"scores", "topk"}, debug);
  sagesla_params all = base(1000, 16);
  check_sequence([all] { return sagesla_select(&all, nullptr); }, {"topk"}, debug);
  sagesla_params none = base(1000, 0);
  check_sequence([none] { return sagesla_select(&none, nullptr); }, {}, debug);
}

static void backward(bool debug) {
  float* const d = (float*)addr(0x90000000);
  sagesla_params p = base();
  p.block_idx = (int32_t*)addr(0x70000000);
  p.workspace_bytes = sagesla_backward_workspace_bytes(&p);
  auto bwd = [d](const sagesla_params& q) { return sagesla_backward(kQ, kK, kV, kOut, d, d, d, d, &q, nullptr); };
  CHECK(bwd(p) == SAGESLA_OK);
  sagesla_params x = p;
  x.block_idx = nullptr;
  CHECK(bwd(x) == SAGESLA_E_NULL);
  CHECK(sagesla_backward(kQ, kK, kV, kOut, d, d, d, nullptr, &p, nullptr) == SAGESLA_E_NULL);  // dw with LINEAR
  CHECK(sagesla_backward(kQ, kK, kV, nullptr, d, d, d, d, &p, nullptr) == SAGESLA_E_NULL);
  CHECK(sagesla_backward(kQ, kK, kV, kOut, (float*)addr(0x90000004), d, d, d, &p, nullptr) == SAGESLA_E_ALIGN);
  x = p;
  x.flags |= SAGESLA_QK_RMSNORM;
  x.q_norm_w = x.k_norm_w = kW;
  CHECK(bwd(x) == SAGESLA_E_NULL);  // dq_norm_w, dk_norm_w required
  x.dq_norm_w = d;
  x.dk_norm_w = (float*)addr(0x90000004);
  CHECK(bwd(x) == SAGESLA_E_ALIGN);
  x.dk_norm_w = d;
  CHECK(bwd(x) == SAGESLA_E_WORKSPACE);  // the norm's buffers need more than p's workspace
  x.workspace_bytes = sagesla_backward_workspace_bytes(&x);
  CHECK(x.workspace_bytes > p.workspace_bytes);
  x.workspace = addr(0x60000010);
  CHECK(bwd(x) == SAGESLA_E_ALIGN);
  x.workspace = kWs;
  check_sequence([=] { return bwd(x); }, {"qk_norm", "linear", "backward_sparse", "backward_linear", "norm_backward"},
                 debug);
  check_sequence([=] { return bwd(p); }, {"linear", "backward_sparse", "backward_linear"}, debug);
  sagesla_params all = base(1000, 16);
  all.block_idx = p.block_idx;
  all.workspace_bytes = sagesla_backward_workspace_bytes(&all);
  check_sequence([=] { return bwd(all); }, {"backward_sparse", "fill"}, debug);
}

static void w8a8(bool debug) {
  void* const x = addr(0xa0000000);
  int8_t* const c8 = (int8_t*)addr(0xb0000000);
  float* const sc = (float*)addr(0xc0000000);
  CHECK(w8a8_quantize(x, 256, 200, 1.f, c8, sc, nullptr) == SAGESLA_E_UNSUPPORTED);
  CHECK(w8a8_quantize(x, 155345, 13824, 1.f, c8, sc, nullptr) == SAGESLA_E_UNSUPPORTED);  // rows * cols >= 2^31
  CHECK(w8a8_quantize(x, (1 << 24) + 1, 128, 1.f, c8, sc, nullptr) == SAGESLA_E_UNSUPPORTED);  // rows > 2^24
  CHECK(w8a8_quantize(x, 0, 256, 1.f, c8, sc, nullptr) == SAGESLA_E_SHAPE);
  CHECK(w8a8_quantize(x, 256, 256, 0.f, c8, sc, nullptr) == SAGESLA_E_SHAPE);
  CHECK(w8a8_quantize(x, 256, 256, 1.5f, c8, sc, nullptr) == SAGESLA_E_SHAPE);
  CHECK(w8a8_quantize(x, 256, 256, NAN, c8, sc, nullptr) == SAGESLA_E_SHAPE);
  CHECK(w8a8_quantize(nullptr, 256, 256, 1.f, c8, sc, nullptr) == SAGESLA_E_NULL);
  CHECK(w8a8_quantize(x, 256, 256, 1.f, c8, (float*)addr(0xc0000004), nullptr) == SAGESLA_E_ALIGN);
  check_sequence([=] { return w8a8_quantize(x, 256, 256, 0.9f, c8, sc, nullptr); }, {"w8a8_quant"}, debug);
  uint16_t* const y = (uint16_t*)addr(0xd0000000);
  CHECK(w8a8_gemm(c8, sc, c8, sc, nullptr, y, 256, 200, 256, nullptr) == SAGESLA_E_UNSUPPORTED);
  CHECK(w8a8_gemm(c8, sc, c8, sc, nullptr, y, 256, 256, 32768 + 128, nullptr) == SAGESLA_E_UNSUPPORTED);
  CHECK(w8a8_gemm(c8, sc, c8, sc, nullptr, y, 155345, 256, 13824, nullptr) == SAGESLA_E_UNSUPPORTED);  // M K >= 2^31
  CHECK(w8a8_gemm(c8, sc, c8, sc, nullptr, y, 256, 155345, 13824, nullptr) == SAGESLA_E_UNSUPPORTED);  // N K >= 2^31
  CHECK(w8a8_gemm(c8, sc, c8, nullptr, nullptr, y, 256, 256, 256, nullptr) == SAGESLA_E_NULL);
  CHECK(w8a8_gemm(c8, sc, c8, sc, addr(0xe0000002), y, 256, 256, 256, nullptr) == SAGESLA_E_ALIGN);
  check_sequence([=] { return w8a8_gemm(c8, sc, c8, sc, nullptr, y, 256, 256, 256, nullptr); }, {"w8a8_gemm"}, debug);
  CHECK(w8a8_workspace_bytes(256, 200) == 0);
  CHECK(w8a8_workspace_bytes(256, 32768 + 128) == 0);
  const size_t ws = w8a8_workspace_bytes(300, 512);
  CHECK(ws >= 300 * 512 + 3 * 4 * sizeof(float));
  CHECK(w8a8_linear(x, c8, sc, nullptr, y, 300, 256, 512, 1.f, kWs, ws - 1, nullptr) == SAGESLA_E_WORKSPACE);
  CHECK(w8a8_linear(x, c8, sc, nullptr, y, 300, 256, 512, 1.f, nullptr, ws, nullptr) == SAGESLA_E_WORKSPACE);
  CHECK(w8a8_linear(x, c8, sc, nullptr, y, 300, 256, 512, 1.f, addr(0x60000040), ws, nullptr) == SAGESLA_E_ALIGN);
  check_sequence([=] { return w8a8_linear(x, c8, sc, nullptr, y, 300, 256, 512, 1.f, kWs, ws, nullptr); },
                 {"w8a8_quant", "w8a8_gemm"}, debug);
}

static void noalloc(bool debug) {
  auto na = [](const sagesla_params& q) { return sagesla_forward_noalloc(kQ, kK, kV, kOut, &q, nullptr); };
  sagesla_params p = base();
  p.workspace = nullptr;  // ignored
  p.workspace_bytes = 0;
  sagesla_params big = base(75600, 118);
  big.H = 40;
  CHECK(sagesla_workspace_bytes(&big) > SAGESLA_NOALLOC_SCRATCH_BYTES);
  stub::reset();
  const int lookups0 = stub::symbol_lookups;
  CHECK(na(big) == SAGESLA_E_WORKSPACE);
  CHECK(stub::symbol_lookups == lookups0 && stub::calls.empty());
  CHECK(sagesla_forward_noalloc(nullptr, kK, kV, kOut, &p, nullptr) == SAGESLA_E_NULL);
  // device lookups fail: reported as HIP errors, nothing launched
  stub::device_code = hipErrorInvalidDevice;
  CHECK(na(p) == SAGESLA_E_HIP && sagesla_last_hip_error() == hipErrorInvalidDevice && stub::calls.empty());
  stub::reset();
  stub::device = 3;
  stub::symbol_code = hipErrorInvalidSymbol;
  CHECK(na(p) == SAGESLA_E_HIP && sagesla_last_hip_error() == hipErrorInvalidSymbol && stub::calls.empty());
  stub::reset();
  stub::device = 64;
  CHECK(na(p) == SAGESLA_E_UNSUPPORTED);
  // success: one address lookup per device, then the cached address; the workspace lies in the scratch array
  stub::reset();
  const int l0 = stub::symbol_lookups;
  CHECK(na(p) == SAGESLA_OK);
  CHECK(stub::symbol_lookups == l0 + 1);
  void* const w0 = stub::workspace_seen;
  CHECK(w0 && (uintptr_t)w0 % 256 == 0);
  stub::reset();
  CHECK(na(p) == SAGESLA_OK && stub::symbol_lookups == l0 + 1 && stub::workspace_seen == w0);
  stub::reset();
  stub::device = 1;
  CHECK(na(p) == SAGESLA_OK && stub::symbol_lookups == l0 + 2);
  stub::reset();
  check_sequence([=] { return na(p); }, {"kmean", "quant", "scores", "topk", "linear", "attn"}, debug);
}

static void thread_local_error() {
  stub::reset();
  stub::fail_at = 0;
  stub::fail_code = hipErrorOutOfMemory;
  sagesla_params p = base();
  CHECK(fwd(p) == SAGESLA_E_HIP);
  CHECK(sagesla_last_hip_error() == hipErrorOutOfMemory);
  int other = -1;
  std::thread t([&] { other = sagesla_last_hip_error(); });
  t.join();
  CHECK(other == 0);
  stub::reset();
  CHECK(fwd(p) == SAGESLA_OK);
  CHECK(sagesla_last_hip_error() == hipErrorOutOfMemory);  // a success does not clear it
}

int main(int argc, char** argv) {
  const bool debug = argc > 1 && strcmp(argv[1], "debug") == 0;
  status_strings();
  validation();
  workspace_sizes();
  forward(debug);
  quantize_select(debug);
  backward(debug);
  w8a8(debug);
  noalloc(debug);
  thread_local_error();
  printf("host ABI checks passed: %d (%s mode)\n", g_checks, debug ? "debug" : "default");
  return 0;
}
