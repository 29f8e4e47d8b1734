// C ABI of the SageSLA forward: host-side validation, workspace plan and launch order.
// The entry points and their contracts are declared in include/sagesla.h.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "internal.h"
#include "sagesla.h"
#include "w8a8.h"

using namespace sagesla;

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
constexpr int kColsumChunk = 512;
constexpr int kMaxN = 1 << 24;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool misaligned(const void* ptr, size_t a) { return ptr && ((uintptr_t)ptr % a) != 0; }

// sizes, block shapes and flags only
sagesla_status check_shape(const sagesla_params* p) {
  if (!p) return SAGESLA_E_NULL;
  if (p->D != kD || p->blk_k != kBlkK || (p->blk_q != 64 && p->blk_q != 128)) return SAGESLA_E_UNSUPPORTED;
  if (p->flags & ~(uint32_t)(SAGESLA_LINEAR | SAGESLA_SMOOTH_K | SAGESLA_USE_GIVEN_MASK | SAGESLA_QUANT_GROUP32 |
                             SAGESLA_QK_RMSNORM))
    return SAGESLA_E_UNSUPPORTED;
  if (p->B < 1 || p->H < 1 || p->N < 1) return SAGESLA_E_SHAPE;
  if ((int64_t)p->B * p->H > 65535) return SAGESLA_E_SHAPE;
  if (p->N > kMaxN) return SAGESLA_E_UNSUPPORTED;
  const int n_kb = (p->N + kBlkK - 1) / kBlkK;
  if (n_kb > kMaxKeyBlocks) return SAGESLA_E_UNSUPPORTED;
  if (p->topk < 0 || p->topk > n_kb) return SAGESLA_E_SHAPE;
  if (!(isfinite(p->sm_scale) && p->sm_scale >= 0.f)) return SAGESLA_E_SHAPE;
  if ((p->flags & SAGESLA_QK_RMSNORM) && !(isfinite(p->norm_eps) && p->norm_eps >= 0.f)) return SAGESLA_E_SHAPE;
  return SAGESLA_OK;
}

// the whole parameter block: shape plus the pointers it carries
sagesla_status check_params(const sagesla_params* p) {
  const sagesla_status st = check_shape(p);
  if (st != SAGESLA_OK) return st;
  if ((p->flags & SAGESLA_LINEAR) && !p->w_proj) return SAGESLA_E_NULL;
  if ((p->flags & SAGESLA_QK_RMSNORM) && (!p->q_norm_w || !p->k_norm_w)) return SAGESLA_E_NULL;
  if (misaligned(p->w_proj, 16) || misaligned(p->q_i8, 16) || misaligned(p->k_i8, 16) ||
      misaligned(p->q_scale, 16) || misaligned(p->k_scale, 16) || misaligned(p->k_mean, 16) ||
      misaligned(p->q_pool, 16) || misaligned(p->k_pool, 16) || misaligned(p->block_idx, 16) ||
      misaligned(p->o_lin, 16) || misaligned(p->q_norm_w, 16) || misaligned(p->k_norm_w, 16) ||
      misaligned(p->q_hat, 16) || misaligned(p->k_hat, 16) || misaligned(p->scores, 16))
    return SAGESLA_E_ALIGN;
  return SAGESLA_OK;
}

// Sizes and placement of every intermediate. With ws == nullptr only the sizes are computed. The backward's plan
// (backward = true) holds only what it reads: the normalized Q and K (with the norm) and its linear branch's fp32
// state table, keep mask and bf16 hi + lo remaining states; the selection comes from the caller.
void make_plan(const sagesla_params* p, unsigned char* ws, Plan* pl, bool backward = false) {
  memset(pl, 0, sizeof(*pl));
  pl->B = p->B;
  pl->H = p->H;
  pl->BH = p->B * p->H;
  pl->N = p->N;
  pl->blk_q = p->blk_q;
  pl->n_qb = (p->N + p->blk_q - 1) / p->blk_q;
  pl->n_kb = (p->N + kBlkK - 1) / kBlkK;
  pl->topk = p->topk;
  pl->smooth = (p->flags & SAGESLA_SMOOTH_K) != 0;
  pl->linear = (p->flags & SAGESLA_LINEAR) != 0;
  pl->given_mask = (p->flags & SAGESLA_USE_GIVEN_MASK) != 0;
  pl->group32 = (p->flags & SAGESLA_QUANT_GROUP32) != 0;
  pl->n_g = (p->N + 31) / 32;
  pl->qk_norm = (p->flags & SAGESLA_QK_RMSNORM) != 0;
  pl->norm_eps = p->norm_eps;
  pl->q_norm_w = p->q_norm_w;
  pl->k_norm_w = p->k_norm_w;
  pl->sm_scale = p->sm_scale > 0.f ? p->sm_scale : 1.f / sqrtf((float)p->D);
  pl->colsum_chunk = kColsumChunk;
  pl->n_colsum_chunks = (p->N + kColsumChunk - 1) / kColsumChunk;
  pl->w_proj = p->w_proj;
  pl->lin_precise = backward;
  const bool lin_active = pl->linear && pl->topk < pl->n_kb;
  pl->states_in_quant = lin_active && !backward;
  const size_t BH = pl->BH, N = pl->N, D = kD, nqb = pl->n_qb, nkb = pl->n_kb;
  size_t off = 0;
  auto take = [&](size_t bytes) -> unsigned char* {
    unsigned char* r = ws ? ws + off : nullptr;
    off += align_up(bytes);
    return r;
  };
  if (pl->qk_norm) {
    pl->q_hat = (uint16_t*)take(BH * N * D * sizeof(uint16_t));
    pl->k_hat = (uint16_t*)take(BH * N * D * sizeof(uint16_t));
  }
  if (!backward) {
    pl->colsum_part = (double*)take(BH * pl->n_colsum_chunks * D * sizeof(double));
    pl->k_mean = (float*)take(BH * D * sizeof(float));
    pl->q_i8 = (int8_t*)take(BH * N * D);
    pl->k_i8 = (int8_t*)take(BH * N * D);
    pl->q_scale = (float*)take(BH * (pl->group32 ? (size_t)pl->n_g : nqb) * sizeof(float));
    pl->k_scale = (float*)take(BH * (pl->group32 ? (size_t)pl->n_g : nkb) * sizeof(float));
    pl->k_norm2 = (int32_t*)take(BH * (pl->group32 ? (size_t)pl->n_g : nkb) * sizeof(int32_t));
    pl->q_pool = (double*)take(BH * nqb * D * sizeof(double));
    pl->k_pool = (double*)take(BH * nkb * D * sizeof(double));
    pl->scores = (double*)take(BH * nqb * nkb * sizeof(double));
    pl->v_img = (unsigned char*)take(BH * nkb * 16384);
    pl->block_idx = (int32_t*)take(BH * nqb * (size_t)pl->topk * sizeof(int32_t));
  }
  if (lin_active) {
    pl->wpt = (uint16_t*)take(D * D * sizeof(uint16_t));
    pl->keep_mask = (uint32_t*)take(BH * (size_t)mask_row_pad(pl->n_qb) * ((nkb + 31) / 32) * sizeof(uint32_t));
    if (backward) {
      pl->state = (float*)take(BH * nkb * kStateX * sizeof(float));
      pl->state_m = (float*)take(BH * nqb * kStateX * sizeof(float));
    } else {
      pl->state16 = (uint16_t*)take(BH * nkb * kStateX * sizeof(uint16_t));
      pl->state_exp = (int32_t*)take(BH * nkb * sizeof(int32_t));
      pl->plane16 = (unsigned char*)take(BH * D * nqb * 256);
      pl->aux16 = (unsigned char*)take(BH * nqb * (size_t)kAuxBytes);
    }
  }
  pl->ws_bytes = off;
  // caller-owned exports replace their workspace slice
  if (p->k_mean) pl->k_mean = p->k_mean;
  if (p->q_i8) pl->q_i8 = p->q_i8;
  if (p->k_i8) pl->k_i8 = p->k_i8;
  if (p->q_scale) pl->q_scale = p->q_scale;
  if (p->k_scale) pl->k_scale = p->k_scale;
  if (p->q_pool) pl->q_pool = p->q_pool;
  if (p->k_pool) pl->k_pool = p->k_pool;
  if (p->block_idx) pl->block_idx = p->block_idx;
  if (p->scores && !backward) pl->scores = p->scores;
  if (pl->qk_norm && p->q_hat) pl->q_hat = (uint16_t*)p->q_hat;
  if (pl->qk_norm && p->k_hat) pl->k_hat = (uint16_t*)p->k_hat;
  pl->o_lin = lin_active ? p->o_lin : nullptr;  // optional export
}

sagesla_status check_workspace(const sagesla_params* p, const Plan& pl) {
  if (p->workspace_bytes < pl.ws_bytes) return SAGESLA_E_WORKSPACE;
  if (!p->workspace) return SAGESLA_E_WORKSPACE;
  if (misaligned(p->workspace, kAlign)) return SAGESLA_E_ALIGN;
  return SAGESLA_OK;
}

sagesla_status hip_status(hipError_t e) {
  if (e == hipSuccess) return SAGESLA_OK;
  g_last_hip_error = (int)e;
  return SAGESLA_E_HIP;
}

// SAGESLA_DEBUG set to anything but "" or "0" (read at the first launch): every kernel launch is followed by a
// synchronization of its stream, so that a fault while the kernel runs is reported as SAGESLA_E_HIP by the entry
// point that launched it, with the launch named on stderr, instead of surfacing at a later call. It blocks the
// host after every launch and cannot be used while the stream is being captured into a graph.
bool debug_sync() {
  static const bool on = [] {
    const char* e = getenv("SAGESLA_DEBUG");
    return e && e[0] && strcmp(e, "0") != 0;
  }();
  return on;
}

// status of a launch (its hipError_t) and, in debug mode, of the kernel's run
sagesla_status launched(hipError_t e, const char* what, hipStream_t s) {
  if (debug_sync()) {
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) fprintf(stderr, "sagesla: %s: %s\n", what, hipGetErrorString(e));
  }
  return hip_status(e);
}

// a kernel launch on stream s (the name of the launcher goes to the debug message)
#define SAGESLA_LAUNCH(s, launcher, ...)                                           \
  do {                                                                             \
    sagesla_status st_ = launched(launcher(__VA_ARGS__), #launcher, (s));          \
    if (st_ != SAGESLA_OK) return st_;                                             \
  } while (0)

// records the caller's timing event of stage `stage` (begin: 0, end: 1) if events were given
sagesla_status mark(const sagesla_params* p, int stage, int end, hipStream_t s) {
  if (!p->events) return SAGESLA_OK;
  void* ev = p->events[2 * stage + end];
  if (!ev) return SAGESLA_OK;
  return hip_status(hipEventRecord((hipEvent_t)ev, s));
}

// the Q and K every step after the optional norm reads: the caller's, or their normalized copies
const void* eff_q(const Plan& pl, const void* q) { return pl.qk_norm ? (const void*)pl.q_hat : q; }
const void* eff_k(const Plan& pl, const void* k) { return pl.qk_norm ? (const void*)pl.k_hat : k; }

sagesla_status run_quantize(const Plan& pl, const void* q_in, const void* k_in, const void* v, hipStream_t s) {
  if (pl.qk_norm) SAGESLA_LAUNCH(s, launch_qk_norm, pl, (const uint16_t*)q_in, (const uint16_t*)k_in, s);
  const void* q = eff_q(pl, q_in);
  const void* k = eff_k(pl, k_in);
  SAGESLA_LAUNCH(s, launch_kmean, pl, (const uint16_t*)k, s);
  SAGESLA_LAUNCH(s, launch_quant, pl, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s);
  return SAGESLA_OK;
}

sagesla_status run_select(const Plan& pl, hipStream_t s) {
  if (pl.topk > 0 && pl.topk < pl.n_kb) SAGESLA_LAUNCH(s, launch_scores, pl, s);
  if (pl.topk > 0) SAGESLA_LAUNCH(s, launch_topk, pl, s);
  return SAGESLA_OK;
}

}  // namespace

extern "C" {

sagesla_status sagesla_validate(const sagesla_params* p) { return check_params(p); }

size_t sagesla_workspace_bytes(const sagesla_params* p) {
  if (check_shape(p) != SAGESLA_OK) return 0;
  Plan pl;
  make_plan(p, nullptr, &pl);
  return pl.ws_bytes;
}

sagesla_status sagesla_quantize(const void* q, const void* k, const sagesla_params* p, void* stream) {
  sagesla_status st = check_params(p);
  if (st != SAGESLA_OK) return st;
  if (!q || !k) return SAGESLA_E_NULL;
  if (misaligned(q, 16) || misaligned(k, 16)) return SAGESLA_E_ALIGN;
  Plan pl;
  make_plan(p, nullptr, &pl);
  if ((st = check_workspace(p, pl)) != SAGESLA_OK) return st;
  make_plan(p, (unsigned char*)p->workspace, &pl);
  return run_quantize(pl, q, k, nullptr, (hipStream_t)stream);
}

sagesla_status sagesla_select(const sagesla_params* p, void* stream) {
  sagesla_status st = check_params(p);
  if (st != SAGESLA_OK) return st;
  Plan pl;
  make_plan(p, nullptr, &pl);
  if ((st = check_workspace(p, pl)) != SAGESLA_OK) return st;
  make_plan(p, (unsigned char*)p->workspace, &pl);
  return run_select(pl, (hipStream_t)stream);
}

sagesla_status sagesla_forward(const void* q, const void* k, const void* v, void* out, const sagesla_params* p,
                               void* stream) {
  sagesla_status st = check_params(p);
  if (st != SAGESLA_OK) return st;
  if (!q || !k || !v || !out) return SAGESLA_E_NULL;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16)) return SAGESLA_E_ALIGN;
  if ((p->flags & SAGESLA_USE_GIVEN_MASK) && p->topk > 0 && !p->block_idx) return SAGESLA_E_NULL;
  Plan pl;
  make_plan(p, nullptr, &pl);
  if ((st = check_workspace(p, pl)) != SAGESLA_OK) return st;
  make_plan(p, (unsigned char*)p->workspace, &pl);
  const hipStream_t s = (hipStream_t)stream;
#define SAGESLA_STEP(expr)                                     \
  do {                                                         \
    if ((st = (expr)) != SAGESLA_OK) return st;                \
  } while (0)
  SAGESLA_STEP(mark(p, SAGESLA_STAGE_QUANTIZE, 0, s));
  SAGESLA_STEP(run_quantize(pl, q, k, v, s));
  SAGESLA_STEP(mark(p, SAGESLA_STAGE_QUANTIZE, 1, s));
  SAGESLA_STEP(mark(p, SAGESLA_STAGE_SELECT, 0, s));
  if (!pl.given_mask) SAGESLA_STEP(run_select(pl, s));
  SAGESLA_STEP(mark(p, SAGESLA_STAGE_SELECT, 1, s));
  SAGESLA_STEP(mark(p, SAGESLA_STAGE_LINEAR, 0, s));
  const bool lin_active = pl.linear && pl.topk < pl.n_kb;
  if (lin_active) {
    SAGESLA_LAUNCH(s, launch_linear, pl, (const uint16_t*)eff_k(pl, k), (const uint16_t*)v, s);
  } else if (p->o_lin) {
    SAGESLA_LAUNCH(s, launch_fill_f32, p->o_lin, (size_t)pl.BH * pl.N * kD, 0.f, s);
  }
  SAGESLA_STEP(mark(p, SAGESLA_STAGE_LINEAR, 1, s));
  SAGESLA_STEP(mark(p, SAGESLA_STAGE_ATTN, 0, s));
  SAGESLA_LAUNCH(s, launch_attn, pl, (const uint16_t*)eff_q(pl, q), (uint16_t*)out, s);
  SAGESLA_STEP(mark(p, SAGESLA_STAGE_ATTN, 1, s));
#undef SAGESLA_STEP
  return SAGESLA_OK;
}

// ---------------------------------------------------------------------------------------------------------
// W8A8 linear layer (include/w8a8.h)
// ---------------------------------------------------------------------------------------------------------
}  // extern "C"

namespace {

constexpr int32_t kW8a8MaxK = 32768;
constexpr int32_t kW8a8MaxRows = 1 << 24;

// rows × cols matrix cut into 128×128 blocks: sizes and limits
sagesla_status w8a8_check_matrix(int32_t rows, int32_t cols) {
  if (rows < 1 || cols < 1) return SAGESLA_E_SHAPE;
  if (cols % 128 != 0 || rows > kW8a8MaxRows || (int64_t)rows * cols >= ((int64_t)1 << 31))
    return SAGESLA_E_UNSUPPORTED;
  return SAGESLA_OK;
}

sagesla_status w8a8_check_gemm(int32_t M, int32_t N, int32_t K) {
  sagesla_status st;
  if ((st = w8a8_check_matrix(M, K)) != SAGESLA_OK) return st;
  if ((st = w8a8_check_matrix(N, K)) != SAGESLA_OK) return st;
  if (N % 128 != 0 || K > kW8a8MaxK) return SAGESLA_E_UNSUPPORTED;
  return SAGESLA_OK;
}

size_t w8a8_scale_count(int32_t rows, int32_t cols) { return (size_t)((rows + 127) / 128) * (cols / 128); }

}  // namespace

extern "C" {

sagesla_status w8a8_quantize(const void* x, int32_t rows, int32_t cols, float clip, int8_t* codes,
                             float* scales, void* stream) {
  sagesla_status st = w8a8_check_matrix(rows, cols);
  if (st != SAGESLA_OK) return st;
  if (!(clip > 0.f && clip <= 1.f)) return SAGESLA_E_SHAPE;
  if (!x || !codes || !scales) return SAGESLA_E_NULL;
  if (misaligned(x, 16) || misaligned(codes, 16) || misaligned(scales, 16)) return SAGESLA_E_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  SAGESLA_LAUNCH(s, launch_w8a8_quant, (const uint16_t*)x, rows, cols, clip, codes, scales, s);
  return SAGESLA_OK;
}

sagesla_status w8a8_gemm(const int8_t* x_i8, const float* x_scale, const int8_t* w_i8, const float* w_scale,
                         const void* bias, void* y, int32_t M, int32_t N, int32_t K, void* stream) {
  sagesla_status st = w8a8_check_gemm(M, N, K);
  if (st != SAGESLA_OK) return st;
  if (!x_i8 || !x_scale || !w_i8 || !w_scale || !y) return SAGESLA_E_NULL;
  if (misaligned(x_i8, 16) || misaligned(x_scale, 16) || misaligned(w_i8, 16) || misaligned(w_scale, 16) ||
      misaligned(bias, 16) || misaligned(y, 16))
    return SAGESLA_E_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  SAGESLA_LAUNCH(s, launch_w8a8_gemm, x_i8, x_scale, w_i8, w_scale, (const uint16_t*)bias, (uint16_t*)y, M, N, K, s);
  return SAGESLA_OK;
}

size_t w8a8_workspace_bytes(int32_t M, int32_t K) {
  if (w8a8_check_matrix(M, K) != SAGESLA_OK || K > kW8a8MaxK) return 0;
  return align_up((size_t)M * K) + align_up(w8a8_scale_count(M, K) * sizeof(float));
}

sagesla_status w8a8_linear(const void* x, const int8_t* w_i8, const float* w_scale, const void* bias, void* y,
                           int32_t M, int32_t N, int32_t K, float clip, void* workspace, size_t workspace_bytes,
                           void* stream) {
  sagesla_status st = w8a8_check_gemm(M, N, K);
  if (st != SAGESLA_OK) return st;
  if (!(clip > 0.f && clip <= 1.f)) return SAGESLA_E_SHAPE;
  if (!x || !w_i8 || !w_scale || !y) return SAGESLA_E_NULL;
  if (misaligned(x, 16) || misaligned(w_i8, 16) || misaligned(w_scale, 16) || misaligned(bias, 16) ||
      misaligned(y, 16))
    return SAGESLA_E_ALIGN;
  if (!workspace || workspace_bytes < w8a8_workspace_bytes(M, K)) return SAGESLA_E_WORKSPACE;
  if (misaligned(workspace, kAlign)) return SAGESLA_E_ALIGN;
  int8_t* x8 = (int8_t*)workspace;
  float* xs = (float*)((unsigned char*)workspace + align_up((size_t)M * K));
  const hipStream_t s = (hipStream_t)stream;
  SAGESLA_LAUNCH(s, launch_w8a8_quant, (const uint16_t*)x, M, K, clip, x8, xs, s);
  SAGESLA_LAUNCH(s, launch_w8a8_gemm, x8, xs, w_i8, w_scale, (const uint16_t*)bias, (uint16_t*)y, M, N, K, s);
  return SAGESLA_OK;
}

// ---------------------------------------------------------------------------------------------------------
// SLA backward for a fixed selection (include/sagesla.h)
// ---------------------------------------------------------------------------------------------------------
}  // extern "C"

namespace {

// the backward's own buffers after its plan's (ws == nullptr: sizes only); returns the total bytes
size_t plan_backward(const Plan& pl, unsigned char* ws, BwdPlan* b) {
  size_t off = pl.ws_bytes;
  auto take = [&](size_t bytes) -> unsigned char* {
    unsigned char* r = ws ? ws + off : nullptr;
    off += align_up(bytes);
    return r;
  };
  const size_t BH = pl.BH, N = pl.N;
  const bool lin_active = pl.linear && pl.topk < pl.n_kb;
  b->lse = (float*)take(BH * N * sizeof(float));
  b->dd = (float*)take(BH * N * sizeof(float));
  b->sel_bits = (uint32_t*)take(BH * pl.n_kb * (size_t)((pl.n_qb + 31) / 32) * sizeof(uint32_t));
  b->sel_bits_q = (uint32_t*)take(BH * pl.n_qb * (size_t)((pl.n_kb + 31) / 32) * sizeof(uint32_t));
  if (lin_active) {
    b->o_l = (float*)take(BH * N * kD * sizeof(float));
    b->dhm = (float*)take(BH * pl.n_qb * (size_t)kStateX * sizeof(float));
    b->keep_t = (uint32_t*)take(BH * (size_t)((pl.n_qb + 31) / 32) * mask_row_pad(pl.n_kb) * sizeof(uint32_t));
    b->dhj = (float*)take(BH * pl.n_kb * (size_t)kStateX * sizeof(float));
    b->dw_part = (float*)take(BH * backward_dw_chunks(pl.N) * kD * kD * sizeof(float));
    b->dw_seg = (float*)take(backward_dw_segments() * kD * kD * sizeof(float));
  }
  if (pl.qk_norm) {
    b->norm_rs = (float*)take((size_t)2 * pl.B * N * 2 * sizeof(float));
    b->norm_part = (float*)take((size_t)2 * pl.B * backward_norm_chunks(pl.N) * pl.H * kD * sizeof(float));
  }
  return off;
}

sagesla_status check_backward(const sagesla_params* p) {
  sagesla_status st = check_params(p);
  if (st != SAGESLA_OK) return st;
  if (p->flags & SAGESLA_QK_RMSNORM) {
    if (!p->dq_norm_w || !p->dk_norm_w) return SAGESLA_E_NULL;
    if (misaligned(p->dq_norm_w, 16) || misaligned(p->dk_norm_w, 16)) return SAGESLA_E_ALIGN;
  }
  if (p->topk > 0 && !p->block_idx) return SAGESLA_E_NULL;
  return SAGESLA_OK;
}

}  // namespace

extern "C" {

size_t sagesla_backward_workspace_bytes(const sagesla_params* p) {
  if (check_shape(p) != SAGESLA_OK) return 0;
  Plan pl;
  make_plan(p, nullptr, &pl, true);
  BwdPlan b{};
  return plan_backward(pl, nullptr, &b);
}

sagesla_status sagesla_backward(const void* q, const void* k, const void* v, const void* dout, float* dq, float* dk,
                                float* dv, float* dw_proj, const sagesla_params* p, void* stream) {
  sagesla_status st = check_backward(p);
  if (st != SAGESLA_OK) return st;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return SAGESLA_E_NULL;
  if ((p->flags & SAGESLA_LINEAR) && !dw_proj) return SAGESLA_E_NULL;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(dout, 16) || misaligned(dq, 16) ||
      misaligned(dk, 16) || misaligned(dv, 16) || misaligned(dw_proj, 16))
    return SAGESLA_E_ALIGN;
  Plan pl;
  make_plan(p, nullptr, &pl, true);
  BwdPlan b{};
  const size_t need = plan_backward(pl, nullptr, &b);
  if (p->workspace_bytes < need || !p->workspace) return SAGESLA_E_WORKSPACE;
  if (misaligned(p->workspace, kAlign)) return SAGESLA_E_ALIGN;
  make_plan(p, (unsigned char*)p->workspace, &pl, true);
  plan_backward(pl, (unsigned char*)p->workspace, &b);
  b.fwd = &pl;
  b.q = (const uint16_t*)q;
  b.k = (const uint16_t*)k;
  b.v = (const uint16_t*)v;
  b.dy = (const uint16_t*)dout;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.dw = dw_proj;
  const hipStream_t s = (hipStream_t)stream;
  if (pl.qk_norm) {  // the attention part runs at the normalized values the forward uses
    SAGESLA_LAUNCH(s, launch_qk_norm, pl, (const uint16_t*)q, (const uint16_t*)k, s);
    b.q = (const uint16_t*)pl.q_hat;
    b.k = (const uint16_t*)pl.k_hat;
  }
  const bool lin_active = pl.linear && pl.topk < pl.n_kb;
  if (lin_active) SAGESLA_LAUNCH(s, launch_linear, pl, b.k, (const uint16_t*)v, s);
  SAGESLA_LAUNCH(s, launch_backward_sparse, b, s);
  if (lin_active) {
    SAGESLA_LAUNCH(s, launch_backward_linear, b, s);
  } else if (dw_proj) {
    SAGESLA_LAUNCH(s, launch_fill_f32, dw_proj, (size_t)kD * kD, 0.f, s);
  }
  if (pl.qk_norm)  // dq, dk hold the gradients at the normalized values: carry them through the norm
    SAGESLA_LAUNCH(s, launch_norm_backward, b, (const uint16_t*)q, (const uint16_t*)k, p->dq_norm_w, p->dk_norm_w, s);
  return SAGESLA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------------------
// The forward without a caller workspace (include/sagesla.h: sagesla_forward_noalloc)
// ---------------------------------------------------------------------------------------------------------
namespace {

constexpr int kMaxDevices = 64;
// The scratch of sagesla_forward_noalloc. In host code this name only stands for the array: its device address on
// a device is looked up there (scratch_address) and only that address is ever passed on.
static __device__ __align__(256) unsigned char scratch[SAGESLA_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];  // per device, after the first lookup

// device address of the scratch array on the current device, looked up once per device
sagesla_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return SAGESLA_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!ptr || misaligned(ptr, kAlign)) return SAGESLA_E_ALIGN;
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return SAGESLA_OK;
}

}  // namespace

extern "C" {

sagesla_status sagesla_forward_noalloc(const void* q, const void* k, const void* v, void* out,
                                       const sagesla_params* p, void* stream) {
  sagesla_status st = check_params(p);
  if (st != SAGESLA_OK) return st;
  if (!q || !k || !v || !out) return SAGESLA_E_NULL;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16)) return SAGESLA_E_ALIGN;
  if ((p->flags & SAGESLA_USE_GIVEN_MASK) && p->topk > 0 && !p->block_idx) return SAGESLA_E_NULL;
  Plan pl;
  make_plan(p, nullptr, &pl);
  if (pl.ws_bytes > SAGESLA_NOALLOC_SCRATCH_BYTES) return SAGESLA_E_WORKSPACE;
  void* ws = nullptr;  // (the first device access of this call)
  if ((st = scratch_address(&ws)) != SAGESLA_OK) return st;
  sagesla_params p2 = *p;
  p2.workspace = ws;
  p2.workspace_bytes = SAGESLA_NOALLOC_SCRATCH_BYTES;
  return sagesla_forward(q, k, v, out, &p2, stream);
}

const char* sagesla_status_str(sagesla_status s) {
  switch (s) {
    case SAGESLA_OK: return "ok";
    case SAGESLA_E_NULL: return "a required pointer is NULL";
    case SAGESLA_E_SHAPE: return "invalid shape or parameter value";
    case SAGESLA_E_UNSUPPORTED: return "unsupported configuration";
    case SAGESLA_E_WORKSPACE: return "workspace missing or too small";
    case SAGESLA_E_ALIGN: return "misaligned pointer";
    case SAGESLA_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int sagesla_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
