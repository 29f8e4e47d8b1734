// Internal declarations shared by the SageSLA host orchestration and its gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sagesla {

constexpr int kD = 128;       // head dim (the only one supported)
constexpr int kBlkK = 64;     // key block
constexpr int kMaxKeyBlocks = 20480;  // n_kb limit of the parameter checks (sizes fixed-size LDS tables)
constexpr int kStateX = kD * kD + kD;  // floats per linear-branch state: H^T (D×D, e-major) then Z (D)
// The forward's remaining state of one query block: H_m^T as an fp16 plane of 128 rows e of 128 columns c, each row
// 256 B in the attention epilogue's swizzled LDS layout, stored row-major over the query blocks of a head
// ([BH][e][n_qb][256 B]: the product kernel writes one e for every query block); and an aux record per query block
// ([BH][n_qb][kAuxBytes]): Z_m (fp32 [D]) then one fp32 factor per row e (a plane row's values times its factor
// give that row of H_m^T). H_m and Z_m share one per-head power-of-two scale.
constexpr int kAuxZ = 0;
constexpr int kAuxF = kD * 4;
constexpr int kAuxBytes = 2 * kD * 4;

// Everything a launch needs, resolved from the parameter block: sizes and where each intermediate lives
// (a caller's export buffer or a slice of the workspace).
struct Plan {
  int B, H, BH, N, blk_q, n_qb, n_kb, topk;
  bool smooth, linear, given_mask;
  bool group32;  // one INT8 scale per 32 tokens (n_g = ceil(N / 32) per (b, h)) instead of one per block
  int n_g;
  bool qk_norm;  // RMSNorm of Q and K over all heads of each token before everything else
  float norm_eps;
  const void* q_norm_w;  // bf16 [H * D]
  const void* k_norm_w;
  uint16_t* q_hat;  // [BH][N][D] bf16 normalized Q and K (workspace or caller export)
  uint16_t* k_hat;
  float sm_scale;
  int colsum_chunk, n_colsum_chunks;
  const void* w_proj;
  // intermediates
  double* colsum_part;  // [BH][n_colsum_chunks][D]
  float* k_mean;        // [BH][D]
  int8_t* q_i8;         // [BH][N][D]
  int8_t* k_i8;
  float* q_scale;       // [BH][n_qb] (or [BH][n_g] with group32)
  float* k_scale;       // [BH][n_kb] (or [BH][n_g] with group32)
  int32_t* k_norm2;     // like k_scale: the largest squared norm of a K code row under that scale
  double* q_pool;       // [BH][n_qb][D]
  double* k_pool;       // [BH][n_kb][D]
  double* scores;       // [BH][n_qb][n_kb]
  unsigned char* v_img; // [BH][n_kb][16384]    per key block: V^T in the attention kernel's LDS layout
  int32_t* block_idx;   // [BH][n_qb][topk]
  uint16_t* wpt;        // [D][D] bf16: W_p^T in MFMA slot order
  uint32_t* keep_mask;  // [BH][ceil(n_kb/32)][mask_row_pad(n_qb)]   bit J set iff key block J is not selected
  // the forward's linear branch (fp16 state table, written by the quantization kernel when states_in_quant)
  bool states_in_quant;
  uint16_t* state16;      // [BH][kStateX / 128][n_kb][128] fp16: block J's state times 2^-e_J
  int32_t* state_exp;     // [BH][n_kb] e_J
  unsigned char* plane16; // [BH][D][n_qb][256 B] rows of the fp16 planes of H_m^T
  unsigned char* aux16;   // [BH][n_qb][kAuxBytes] Z_m and the plane rows' factors
  // the backward's linear branch (lin_precise: fp32 state table, remaining state as bf16 hi + lo planes)
  bool lin_precise;
  float* state;         // [BH][kStateX / 128][n_kb][128]   per-block states, tiles of 128 columns
  float* state_m;       // [BH][n_qb][kStateX]   remaining (non-selected) state per query block
  float* o_lin;         // [BH][N][D] optional export (caller-owned), written by the attention kernel
  size_t ws_bytes;
};

// K0: RMSNorm of Q and K per token over all heads (writes p.q_hat, p.k_hat)
hipError_t launch_qk_norm(const Plan& p, const uint16_t* q, const uint16_t* k, hipStream_t s);
// K1: K-mean smoothing, per-block INT8 quantization and block mean pooling
hipError_t launch_kmean(const Plan& p, const uint16_t* k, hipStream_t s);
// (v may be null: then no V^T images are written; with v and states_in_quant the key-block workgroups also write
// the forward's linear-branch state table, state16 and state_exp)
hipError_t launch_quant(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v, hipStream_t s);
// K2: pooled block scores and top-k selection
hipError_t launch_scores(const Plan& p, hipStream_t s);
hipError_t launch_topk(const Plan& p, hipStream_t s);
// K4: linear branch (block states, sum over the unselected blocks, contraction with phi(Q) and W_p): the forward's
// remaining state (plane16, aux16) from the fp16 table launch_quant wrote, or with lin_precise the backward's fp32
// table and remaining state (state, state_m)
hipError_t launch_linear(const Plan& p, const uint16_t* k, const uint16_t* v, hipStream_t s);
// K3: block-sparse INT8 attention, epilogue adds the linear branch and writes bf16
hipError_t launch_attn(const Plan& p, const uint16_t* q, uint16_t* out, hipStream_t s);
// W8A8 linear layer: 128×128 block quantizer and the block-scaled INT8 product (Y bf16 [M][N])
hipError_t launch_w8a8_quant(const uint16_t* x, int rows, int cols, float clip, int8_t* codes, float* scales,
                             hipStream_t s);
hipError_t launch_w8a8_gemm(const int8_t* x8, const float* xs, const int8_t* w8, const float* ws,
                            const uint16_t* bias, uint16_t* y, int M, int N, int K, hipStream_t s);
// SLA backward for a fixed selection: buffers on top of a forward Plan (whose linear-branch state it reuses)
struct BwdPlan {
  const Plan* fwd;
  const uint16_t *q, *k, *v, *dy;  // bf16 [BH][N][D]
  float *dq, *dk, *dv, *dw;        // outputs: fp32 [BH][N][D], dW_p fp32 [D][D]
  float* lse;                      // [BH][N] base-2 log-sum-exp of each row's selected scores
  float* dd;                       // [BH][N] D_i = sum_j P_ij dP_ij
  uint32_t* sel_bits;              // [BH][n_kb][ceil(n_qb/32)]: bit I of key block J = I selected J
  uint32_t* sel_bits_q;            // [BH][n_qb][ceil(n_kb/32)]: bit J of query block I = I selected J
  float* o_l;                      // [BH][N][D] linear-branch output before W_p
  float* dhm;                      // [BH][kStateX / 128][n_qb][128] per query block dH_m (row c = column group c) then dZ_m
  uint32_t* keep_t;                // [BH][ceil(n_qb/32)][mask_row_pad(n_kb)]: bit I of key block J = I did not select J
  float* dhj;                      // [BH][n_kb] records: dH_J as bf16 hi and lo planes (row c), then dZ_J fp32
  float* dw_part;                  // [BH][n_chunks][D][D]
  float* dw_seg;                   // [backward_dw_segments()][D][D]
  float* norm_rs;                  // with the norm: [2][B][N][2] r and s of every token of Q and K
  float* norm_part;                // with the norm: [2][B][backward_norm_chunks(N)][H*D] weight-gradient partials
};
hipError_t launch_backward_sparse(const BwdPlan& b, hipStream_t s);
hipError_t launch_backward_linear(const BwdPlan& b, hipStream_t s);
size_t backward_dw_chunks(int N);
size_t backward_dw_segments();
size_t backward_norm_chunks(int N);
hipError_t launch_norm_backward(const BwdPlan& b, const uint16_t* q_raw, const uint16_t* k_raw, float* dwq,
                                float* dwk, hipStream_t s);
// fills (graph-capture friendly replacements for memset)
hipError_t launch_fill_f32(float* dst, size_t n, float val, hipStream_t s);
// dynamic LDS of the kernels that size it at run time
size_t topk_lds_bytes(int n_kb);
// query-block rows of the keep mask, padded for the linear-branch product's chunks
int mask_row_pad(int n_qb);
// out[r] = sum over i of mask bit (r, i) times table row i, for every record column: table fp32
// [BH][kStateX / 128][n_in][128], mask [BH][ceil(n_in/32)][pad] (bit i % 32 of word i / 32 of row r), out in the
// remaining-state record format (bf16 hi and lo planes of the first D*D columns, then fp32 columns), [BH][n_out]
hipError_t launch_state_sum(const float* table, const uint32_t* mask, float* out, int n_out, int n_in, int pad, int BH,
                            hipStream_t s);

}  // namespace sagesla
