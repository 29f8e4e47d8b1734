// SLA backward for a fixed block selection (gfx950).
//
// "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn) makes SLA trainable (§三(二); the model is
// fine-tuned with it, §四 step 1). The gradient here is that of the float forward for the given selection:
// out = O_s + O_l W_p, O_s the softmax attention over the selected key blocks with scores q.k * sm_scale, O_l the
// elu+1 linear attention over the unselected blocks; INT8 quantization passes straight through and the K-mean
// shift, which leaves every softmax row unchanged, drops out.
//
// Sparse branch (bf16 MFMA, fp32 accumulation; P and dS enter the products as bf16 hi + lo pairs):
//   kb_sel     bitmap [BH][n_kb][ceil(n_qb/32)]: bit I of key block J = J is selected by query block I
//   kb_q       per query block: pass 1 the log-sum-exp of every row (base 2) and D_i = sum_j P_ij dP_ij, both
//              online; pass 2 dS = P (dP - D) and dQ = dS K sm_scale; writes LSE, D and dQ
//   kb_kv      per key block, over the query blocks that selected it: dV = P^T dY, dK = dS^T Q sm_scale
// Linear branch (fp32 VALU tiles), after the forward's remaining-state product (H_m, Z_m per query block):
//   kb_lin_q   per query block: O_l, dO_l = dY W_p^T, dnum = dO_l / den, dden = -(dO_l . O_l) / den,
//              dQ += (dnum H_m^T + dden Z_m) * phi'(q), and the block's dH_m = phi(Q)^T dnum, dZ_m = phi(Q)^T dden
//   kb_lin_sum per key block J: dH_J, dZ_J = the sums of dH_m, dZ_m over the query blocks that did not select J
//   kb_lin_k   per key block: dK += (V dH_J^T + dZ_J) * phi'(k), dV += phi(K) dH_J
//   kb_dw      dW_p = sum over all rows of O_l^T dY (per-chunk partials, then a fixed-order sum)
// Every sum has a fixed order; no atomics touch floating-point data.
#include "device_common.h"
#include "internal.h"
#include "lin_common.h"

namespace sagesla {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLd128 = kD + 8;  // LDS row stride (bf16 elements) of 128-wide rows: 272 B, conflict-free reads
constexpr int kLd64 = 64 + 8;   // of 64-wide rows: 144 B

// acc[32x32] += A[32 rows][K] . B[32 rows][K]^T with A, B bf16 row-major in LDS (row strides lda, ldb elements).
// Result layout: lane l holds column l % 32 (a row of B) and rows 8 (r/4) + 4 (l/32) + r%4 (rows of A).
__device__ __forceinline__ v16f mma_nt(const __bf16* A, int lda, const __bf16* B, int ldb, int K, v16f c) {
  const int l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const v8bf a = *(const v8bf*)(A + r * lda + k0 + 8 * g);
    const v8bf b = *(const v8bf*)(B + r * ldb + k0 + 8 * g);
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  return c;
}

__device__ __forceinline__ int acc_row(int r) { return 8 * (r >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (r & 3); }

__device__ __forceinline__ __bf16 to_bf16(float x) { return __builtin_bit_cast(__bf16, (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu)); }
__device__ __forceinline__ float from_bf16(__bf16 x) { return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, x) << 16); }

// rows [r0, r0 + nrows) of a [N][128] bf16 head into LDS rows of stride ld (rows past nvalid are zero); 256 threads
template <int NT>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ src, int r0, int nrows, int nvalid,
                                          __bf16* dst, int ld) {
  for (int u = threadIdx.x; u < nrows * 16; u += NT) {
    const int rr = u >> 4, c8 = (u & 15) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rr < nvalid) v = *(const uint4*)(src + (size_t)(r0 + rr) * kD + c8);
    *(uint4*)(dst + rr * ld + c8) = v;
  }
}

// the same rows transposed: dst[c][rr] (row stride ld), c < 128
template <int NT>
__device__ __forceinline__ void load_rows_t(const uint16_t* __restrict__ src, int r0, int nrows, int nvalid,
                                            __bf16* dst, int ld) {
  for (int u = threadIdx.x; u < nrows * 16; u += NT) {
    const int rr = u >> 4, c8 = (u & 15) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rr < nvalid) v = *(const uint4*)(src + (size_t)(r0 + rr) * kD + c8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      dst[(c8 + e) * ld + rr] = __builtin_bit_cast(__bf16, (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu)));
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------------------------
// kb_sel: grid (n_qb, BH), 64 threads. Sets bit I of word [bh][J][I / 32] for every listed J (atomic OR: the
// result does not depend on the order).
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void kb_sel(const int32_t* __restrict__ idx, uint32_t* __restrict__ bits, int n_qb,
                                             int n_kb, int topk, int n_qbw) {
  const int I = blockIdx.x, bh = blockIdx.y;
  const int32_t* row = idx + ((size_t)bh * n_qb + I) * topk;
  for (int t = threadIdx.x; t < topk; t += 64) {
    const int J = min(max(row[t], 0), n_kb - 1);
    atomicOr(&bits[((size_t)bh * n_kb + J) * n_qbw + (I >> 5)], 1u << (I & 31));
  }
}

// ---------------------------------------------------------------------------------------------------------
// kb_q: grid (n_qb, BH), 256 threads (4 waves x 32 query rows). Scores are computed transposed, S^T = K Q^T, so
// each lane owns one query row: row maxima and sums are in-lane plus the partner lane l ^ 32.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kb_q(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                            const uint16_t* __restrict__ v, const uint16_t* __restrict__ dy,
                                            const int32_t* __restrict__ idx, float* __restrict__ lse_out,
                                            float* __restrict__ d_out, float* __restrict__ dq, int N, int n_qb,
                                            int n_kb, int topk, int blk_q, float sm_scale) {
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* sQ = (__bf16*)smem;             // [128][kLd128]
  __bf16* sdY = sQ + 128 * kLd128;        // [128][kLd128]
  __bf16* sK = sdY + 128 * kLd128;        // [64][kLd128]
  __bf16* sV = sK + 64 * kLd128;          // [64][kLd128]
  __bf16* sKt = sV + 64 * kLd128;         // [128][kLd64]   K_J^T
  __bf16* sSh = sKt + 128 * kLd64;        // [128][kLd64]   dS hi
  __bf16* sSl = sSh + 128 * kLd64;        // [128][kLd64]   dS lo
  const int I = blockIdx.x, bh = blockIdx.y;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, lr = l & 31;
  const int r0 = I * blk_q, nq = min(blk_q, N - r0);
  const uint16_t* qh = q + (size_t)bh * N * kD;
  const uint16_t* kh = k + (size_t)bh * N * kD;
  const uint16_t* vh = v + (size_t)bh * N * kD;
  const uint16_t* dyh = dy + (size_t)bh * N * kD;
  const int32_t* row = idx + ((size_t)bh * n_qb + I) * topk;
  load_rows<256>(qh, r0, 128, min(nq, 128), sQ, kLd128);
  load_rows<256>(dyh, r0, 128, min(nq, 128), sdY, kLd128);
  const bool wave_live = 32 * w < nq;  // the wave's rows exist (blk_q 64: waves 2, 3 idle but still sync)
  const float c2 = sm_scale * kLog2e;
  const int i_loc = 32 * w + lr;  // this lane's query row in the block
  // a key block appears once even if listed twice
  auto listed_before = [&](int t, int J) {
    for (int u = 0; u < t; ++u)
      if (min(max(row[u], 0), n_kb - 1) == J) return true;
    return false;
  };
  auto load_kv = [&](int J, bool with_v, bool with_kt) {
    __syncthreads();  // the previous block's tiles are no longer read
    const int nv = min(64, N - J * 64);
    load_rows<256>(kh, J * 64, 64, nv, sK, kLd128);
    if (with_v) load_rows<256>(vh, J * 64, 64, nv, sV, kLd128);
    if (with_kt) load_rows_t<256>(kh, J * 64, 64, nv, sKt, kLd64);
    __syncthreads();
    return nv;
  };
  // S^T (and dP^T) tiles of this wave: st[t] holds keys 32 t + acc_row(r) of query i_loc
  auto scores = [&](v16f (&st)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) st[t] = mma_nt(sK + 32 * t * kLd128, kLd128, sQ + 32 * w * kLd128, kLd128, kD, (v16f){});
  };
  auto dpt = [&](v16f (&dp)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) dp[t] = mma_nt(sV + 32 * t * kLd128, kLd128, sdY + 32 * w * kLd128, kLd128, kD, (v16f){});
  };
  __syncthreads();

  // pass 1, online per row: m = max of s * c2, l = sum of 2^(s c2 - m) and u = sum of 2^(s c2 - m) dP, both rescaled
  // when m grows; then LSE = m + log2(l) and D = u / l = sum_j P_ij dP_ij
  float m = -INFINITY, lsum = 0.f, usum = 0.f;
  for (int t = 0; t < topk; ++t) {
    const int J = min(max(row[t], 0), n_kb - 1);
    if (listed_before(t, J)) continue;
    const int nv = load_kv(J, true, false);
    v16f st[2], dp[2];
    scores(st);
    dpt(dp);
    if (!wave_live) continue;
    float bm = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * tt + acc_row(r) < nv) bm = fmaxf(bm, st[tt][r] * c2);
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m, bm);
    float ps = 0.f, pu = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * tt + acc_row(r) < nv) {
          const float e = __builtin_amdgcn_exp2f(st[tt][r] * c2 - mn);
          ps += e;
          pu = fmaf(e, dp[tt][r], pu);
        }
    ps += __shfl_xor(ps, 32);
    pu += __shfl_xor(pu, 32);
    const float sc = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    lsum = lsum * sc + ps;
    usum = usum * sc + pu;
    m = mn;
  }
  const float lse = (lsum > 0.f) ? m + __log2f(lsum) : 0.f;  // no selected key: every P is 0 below
  const float dsum = (lsum > 0.f) ? usum / lsum : 0.f;
  if (wave_live && l < 32 && i_loc < nq) {
    lse_out[(size_t)bh * N + r0 + i_loc] = lse;
    d_out[(size_t)bh * N + r0 + i_loc] = dsum;
  }

  // pass 2: dS = P (dP - D) into LDS (rows i, keys j) as hi + lo, then dQ^T tiles += K^T-rows . dS-rows
  v16f acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = (v16f){};
  for (int t = 0; t < topk; ++t) {
    const int J = min(max(row[t], 0), n_kb - 1);
    if (listed_before(t, J)) continue;
    const int nv = load_kv(J, true, true);
    v16f st[2], dp[2];
    scores(st);
    dpt(dp);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        float hv[4], lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = wave_live && 32 * tt + acc_row(r + e) < nv;
          const float p = ok ? __builtin_amdgcn_exp2f(st[tt][r + e] * c2 - lse) : 0.f;
          const float ds = p * (dp[tt][r + e] - dsum);
          hv[e] = from_bf16(to_bf16(ds));
          lv[e] = ds - hv[e];
        }
        const int j0 = 32 * tt + acc_row(r);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sSh[i_loc * kLd64 + j0 + e] = to_bf16(hv[e]);
          sSl[i_loc * kLd64 + j0 + e] = to_bf16(lv[e]);
        }
      }
    // this wave reads back only its own dS rows: a wave-level ordering of its LDS writes suffices
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[u] = mma_nt(sKt + 32 * u * kLd64, kLd64, sSh + 32 * w * kLd64, kLd64, 64, acc[u]);
      acc[u] = mma_nt(sKt + 32 * u * kLd64, kLd64, sSl + 32 * w * kLd64, kLd64, 64, acc[u]);
    }
  }
  // acc[u][r] = dQ^T[d = 32 u + acc_row(r)][i = i_loc] (unscaled)
  if (wave_live && i_loc < nq) {
    float* dst = dq + ((size_t)bh * N + r0 + i_loc) * kD;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 16; r += 4)
        *(float4*)(dst + 32 * u + acc_row(r)) =
            make_float4(acc[u][r] * sm_scale, acc[u][r + 1] * sm_scale, acc[u][r + 2] * sm_scale, acc[u][r + 3] * sm_scale);
  }
}

// ---------------------------------------------------------------------------------------------------------
// kb_kv: grid (n_kb, BH), 256 threads: wave w takes keys 32 (w % 2) .. +31 and rows 32 (w / 2) .. +31 of each
// 64-row half of a query block. For every query block I that selected J (bitmap): S = Q K^T and dP = dY V^T
// tiles with the keys as columns (lane = key), P and dS written transposed (rows = keys) to LDS as hi + lo, then
// dV^T += dY^T-rows . P^T-rows and dK^T += Q^T-rows . dS^T-rows over the wave's 32 rows. The two waves of a key
// tile then hold partial sums over complementary rows, added in a fixed order at the end.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kb_kv(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                             const uint16_t* __restrict__ v, const uint16_t* __restrict__ dy,
                                             const uint32_t* __restrict__ bits, const float* __restrict__ lse_in,
                                             const float* __restrict__ d_in, float* __restrict__ dk,
                                             float* __restrict__ dv, int N, int n_qb, int n_kb, int n_qbw, int blk_q,
                                             float sm_scale) {
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* sQ = (__bf16*)smem;       // [64][kLd128]   64 query rows
  __bf16* sdY = sQ + 64 * kLd128;   // [64][kLd128]
  __bf16* sQt = sdY + 64 * kLd128;  // [128][kLd64]   Q^T of those rows
  __bf16* sdYt = sQt + 128 * kLd64; // [128][kLd64]
  __bf16* sK = sdYt + 128 * kLd64;  // [64][kLd128]
  __bf16* sV = sK + 64 * kLd128;    // [64][kLd128]
  __bf16* sPh = sV + 64 * kLd128;   // [64 keys][kLd64] P^T hi
  __bf16* sPl = sPh + 64 * kLd64;
  __bf16* sDh = sPl + 64 * kLd64;   // dS^T hi
  __bf16* sDl = sDh + 64 * kLd64;
  float* sL = (float*)(sDl + 64 * kLd64);  // [64] LSE of the rows
  float* sDd = sL + 64;                    // [64] D of the rows
  const int J = blockIdx.x, bh = blockIdx.y;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, lr = l & 31;
  const int kt = w & 1, ch = w >> 1;  // key tile, row chunk
  const int nk = min(64, N - J * 64);
  const uint16_t* qh = q + (size_t)bh * N * kD;
  const uint16_t* dyh = dy + (size_t)bh * N * kD;
  load_rows<256>(k + (size_t)bh * N * kD, J * 64, 64, nk, sK, kLd128);
  load_rows<256>(v + (size_t)bh * N * kD, J * 64, 64, nk, sV, kLd128);
  const float c2 = sm_scale * kLog2e;
  const int j_loc = 32 * kt + lr;
  v16f accv[4], acck[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) accv[u] = acck[u] = (v16f){};
  const uint32_t* jb = bits + ((size_t)bh * n_kb + J) * n_qbw;
  for (int wd = 0; wd < n_qbw; ++wd) {
    uint32_t word = jb[wd];
    while (word) {
      const int I = 32 * wd + __builtin_ctz(word);
      word &= word - 1;
      const int q0 = I * blk_q, nq = min(blk_q, N - q0);
      for (int h0 = 0; h0 < nq; h0 += 64) {
        const int nh = min(64, nq - h0);
        __syncthreads();  // the previous half's tiles are no longer read
        load_rows<256>(qh, q0 + h0, 64, nh, sQ, kLd128);
        load_rows<256>(dyh, q0 + h0, 64, nh, sdY, kLd128);
        load_rows_t<256>(qh, q0 + h0, 64, nh, sQt, kLd64);
        load_rows_t<256>(dyh, q0 + h0, 64, nh, sdYt, kLd64);
        if (threadIdx.x < 64) {
          const int ii = threadIdx.x;
          sL[ii] = ii < nh ? lse_in[(size_t)bh * N + q0 + h0 + ii] : 0.f;
          sDd[ii] = ii < nh ? d_in[(size_t)bh * N + q0 + h0 + ii] : 0.f;
        }
        __syncthreads();
        const v16f s = mma_nt(sQ + 32 * ch * kLd128, kLd128, sK + 32 * kt * kLd128, kLd128, kD, (v16f){});
        const v16f dp = mma_nt(sdY + 32 * ch * kLd128, kLd128, sV + 32 * kt * kLd128, kLd128, kD, (v16f){});
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ii = 32 * ch + acc_row(r);
          const bool ok = ii < nh;
          const float p = ok ? __builtin_amdgcn_exp2f(s[r] * c2 - sL[ii]) : 0.f;
          const float ds = p * (dp[r] - sDd[ii]);
          const float ph = from_bf16(to_bf16(p)), dh = from_bf16(to_bf16(ds));
          sPh[j_loc * kLd64 + ii] = to_bf16(ph);
          sPl[j_loc * kLd64 + ii] = to_bf16(p - ph);
          sDh[j_loc * kLd64 + ii] = to_bf16(dh);
          sDl[j_loc * kLd64 + ii] = to_bf16(ds - dh);
        }
        // each wave reads back only the P^T / dS^T entries it wrote (its keys, its 32 rows)
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        const int i0 = 32 * ch;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          accv[u] = mma_nt(sdYt + 32 * u * kLd64 + i0, kLd64, sPh + 32 * kt * kLd64 + i0, kLd64, 32, accv[u]);
          accv[u] = mma_nt(sdYt + 32 * u * kLd64 + i0, kLd64, sPl + 32 * kt * kLd64 + i0, kLd64, 32, accv[u]);
          acck[u] = mma_nt(sQt + 32 * u * kLd64 + i0, kLd64, sDh + 32 * kt * kLd64 + i0, kLd64, 32, acck[u]);
          acck[u] = mma_nt(sQt + 32 * u * kLd64 + i0, kLd64, sDl + 32 * kt * kLd64 + i0, kLd64, 32, acck[u]);
        }
      }
    }
  }
  // acc[u][r] = partial X^T[d = 32 u + acc_row(r)][key j_loc] over the rows of chunk ch: chunk 1 hands its sums
  // to chunk 0 through LDS (the row tiles are free now), which adds them (chunk 0 first) and stores
  __syncthreads();
  float* sX = (float*)smem;  // [2 key tiles][2 (dV, dK)][4 u][16 r][64 lanes]
  if (ch == 1) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sX[(((kt * 2 + 0) * 4 + u) * 16 + r) * 64 + l] = accv[u][r];
        sX[(((kt * 2 + 1) * 4 + u) * 16 + r) * 64 + l] = acck[u][r];
      }
  }
  __syncthreads();
  if (ch == 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        accv[u][r] += sX[(((kt * 2 + 0) * 4 + u) * 16 + r) * 64 + l];
        acck[u][r] += sX[(((kt * 2 + 1) * 4 + u) * 16 + r) * 64 + l];
      }
    if (j_loc < nk) {
      float* dvr = dv + ((size_t)bh * N + J * 64 + j_loc) * kD;
      float* dkr = dk + ((size_t)bh * N + J * 64 + j_loc) * kD;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          *(float4*)(dvr + 32 * u + acc_row(r)) = make_float4(accv[u][r], accv[u][r + 1], accv[u][r + 2], accv[u][r + 3]);
          *(float4*)(dkr + 32 * u + acc_row(r)) = make_float4(acck[u][r] * sm_scale, acck[u][r + 1] * sm_scale,
                                                              acck[u][r + 2] * sm_scale, acck[u][r + 3] * sm_scale);
        }
    }
  }
}

// ---------------------------------------------------------------------------------------------------------
// fp32 VALU tile products for the linear branch: C[M][128] (+)= A[M][K] B[K][128], A and B in LDS with arbitrary
// strides (so transposed operands are read in place). 256 threads: thread (ty = t / 16, tx = t % 16) computes rows
// ty + 16 a (a < M / 16) and columns tx + 16 b (b < 8).
// ---------------------------------------------------------------------------------------------------------
template <int M>
struct VTile {
  float c[M / 16][8];
};

template <int M>
__device__ __forceinline__ void vgemm(VTile<M>& C, const float* A, int a_r, int a_k, const float* B, int b_k, int b_c,
                                      int K) {
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  for (int kk = 0; kk < K; ++kk) {
    float av[M / 16], bv[8];
#pragma unroll
    for (int a = 0; a < M / 16; ++a) av[a] = A[(ty + 16 * a) * a_r + kk * a_k];
#pragma unroll
    for (int b = 0; b < 8; ++b) bv[b] = B[kk * b_k + (tx + 16 * b) * b_c];
#pragma unroll
    for (int a = 0; a < M / 16; ++a)
#pragma unroll
      for (int b = 0; b < 8; ++b) C.c[a][b] = fmaf(av[a], bv[b], C.c[a][b]);
  }
}

template <int M>
__device__ __forceinline__ void vzero(VTile<M>& C) {
#pragma unroll
  for (int a = 0; a < M / 16; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) C.c[a][b] = 0.f;
}

__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : __builtin_amdgcn_exp2f(x * kLog2e); }

// H_m[c][e] of query block I from the remaining-state record (bf16 hi + lo planes of H_m^T, then Z_m fp32)
__device__ __forceinline__ void load_state(const float* state_m, size_t rec, float* sH, float* sZ) {
  const unsigned char* base = (const unsigned char*)state_m + rec;
  for (int u = threadIdx.x; u < kD * kD; u += 256) {
    const int e = u >> 7, c = u & 127;
    const uint16_t hi = *(const uint16_t*)(base + out_off(e, c));
    const uint16_t lo = *(const uint16_t*)(base + 32768 + out_off(e, c));
    sH[c * kD + e] = __uint_as_float((uint32_t)hi << 16) + __uint_as_float((uint32_t)lo << 16);
  }
  for (int u = threadIdx.x; u < kD; u += 256) sZ[u] = *(const float*)(base + 65536 + 4 * u);
}

// ---------------------------------------------------------------------------------------------------------
// kb_lin_q: grid (n_qb, BH), 256 threads; dynamic LDS: two 128x128 fp32 planes (A, B) + vectors.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kb_lin_q(const uint16_t* __restrict__ q, const uint16_t* __restrict__ dy,
                                                const uint16_t* __restrict__ w_proj, const float* __restrict__ state_m,
                                                float* __restrict__ o_l, float* __restrict__ dq,
                                                float* __restrict__ dhm, int N, int n_qb, int blk_q) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* pA = (float*)smem;      // [128][128]
  float* pB = pA + kD * kD;      // [128][128]
  float* sZ = pB + kD * kD;      // [128]
  float* sDen = sZ + kD;         // [128]
  float* sDd = sDen + kD;        // [128]
  float* sRed = sDd + kD;        // [16][128]
  const int I = blockIdx.x, bh = blockIdx.y, t = threadIdx.x, ty = t >> 4, tx = t & 15;
  const int r0 = I * blk_q, nq = min(blk_q, N - r0);
  const size_t rec = ((size_t)bh * n_qb + I) * (size_t)kStateX * 4;
  const uint16_t* qr = q + ((size_t)bh * N + r0) * kD;
  const uint16_t* dyr = dy + ((size_t)bh * N + r0) * kD;
  // phase A: pA = phi(Q) [i][c] (rows past nq are 0), pB = H_m [c][e]; num = phi(Q) H_m, den = phi(Q) . Z_m
  for (int u = t; u < kD * kD; u += 256) {
    const int i = u >> 7;
    pA[u] = i < nq ? phi_f(bf16_lo(qr[u])) : 0.f;
  }
  load_state(state_m, rec, pB, sZ);
  __syncthreads();
  for (int i = t; i < kD; i += 256) {
    float s = 0.f;
    for (int c = 0; c < kD; ++c) s = fmaf(pA[i * kD + c], sZ[c], s);
    sDen[i] = s;
  }
  VTile<128> num;
  vzero(num);
  vgemm(num, pA, kD, 1, pB, kD, 1, kD);
  __syncthreads();
  float ol[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int i = ty + 16 * a;
      ol[a][b] = i < nq ? num.c[a][b] / sDen[i] : 0.f;
    }
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int i = ty + 16 * a;
    if (i < nq)
#pragma unroll
      for (int b = 0; b < 8; ++b) o_l[((size_t)bh * N + r0 + i) * kD + tx + 16 * b] = ol[a][b];
  }
  __syncthreads();
  // phase B: pA = dY [i][f], pB = W_p [e][f]; dO_l = dY W_p^T; dnum = dO_l / den; dden = -(dO_l . O_l) / den
  for (int u = t; u < kD * kD; u += 256) {
    pA[u] = (u >> 7) < nq ? bf16_lo(dyr[u]) : 0.f;
    pB[u] = bf16_lo(w_proj[u]);
  }
  __syncthreads();
  VTile<128> dol;
  vzero(dol);
  vgemm(dol, pA, kD, 1, pB, 1, kD, kD);  // B[kk = f][col = e] = W_p[e][f]
  float part[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    part[a] = 0.f;
#pragma unroll
    for (int b = 0; b < 8; ++b) part[a] = fmaf(dol.c[a][b], ol[a][b], part[a]);
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) sRed[tx * kD + ty + 16 * a] = part[a];
  __syncthreads();
  if (t < kD) {
    float s = 0.f;
    for (int x = 0; x < 16; ++x) s += sRed[x * kD + t];
    sDd[t] = t < nq ? -s / sDen[t] : 0.f;
  }
  __syncthreads();
  // phase C: pA = dnum [i][e]; pB = H_m [c][e] again; dphi_q = dnum H_m^T + dden Z_m; dQ += dphi_q * phi'(q)
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int i = ty + 16 * a;
      pA[i * kD + tx + 16 * b] = i < nq ? dol.c[a][b] / sDen[i] : 0.f;
    }
  load_state(state_m, rec, pB, sZ);
  __syncthreads();
  VTile<128> dpq;
  vzero(dpq);
  vgemm(dpq, pA, kD, 1, pB, 1, kD, kD);  // B[kk = e][col = c] = H_m[c][e]
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int i = ty + 16 * a;
    if (i < nq)
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int c = tx + 16 * b;
        float* d = dq + ((size_t)bh * N + r0 + i) * kD + c;
        *d += (dpq.c[a][b] + sDd[i] * sZ[c]) * dphi(bf16_lo(qr[i * kD + c]));
      }
  }
  __syncthreads();
  // phase D: pB = phi(Q) [i][c]; dH_m = phi(Q)^T dnum -> C[c][e] = sum_i pB[i][c] pA[i][e]; dZ_m = phi(Q)^T dden
  for (int u = t; u < kD * kD; u += 256) {
    const int i = u >> 7;
    pB[u] = i < nq ? phi_f(bf16_lo(qr[u])) : 0.f;
  }
  __syncthreads();
  VTile<128> dh;
  vzero(dh);
  vgemm(dh, pB, 1, kD, pA, kD, 1, kD);  // A[row = c][kk = i] = phi(Q)[i][c]
  float* out = dhm + ((size_t)bh * n_qb + I) * kStateX;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) out[(ty + 16 * a) * kD + tx + 16 * b] = dh.c[a][b];
  if (t < kD) {
    float s = 0.f;
    for (int i = 0; i < kD; ++i) s = fmaf(pB[i * kD + t], sDd[i], s);
    out[kD * kD + t] = s;
  }
}

// ---------------------------------------------------------------------------------------------------------
// kb_lin_sum: grid (ceil(kStateX / 256), ceil(n_kb / 64), BH), 256 threads. Thread t owns column x = 256 bx + t
// of the key blocks J0 .. J0+63 and adds dH_m[I][x] over the query blocks I in ascending order whenever J is not
// selected by I (the keep mask of the forward's linear stage).
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kb_lin_sum(const float* __restrict__ dhm, const uint32_t* __restrict__ keep,
                                                  float* __restrict__ dhj, int n_qb, int n_kb, int n_kbw, int qpad) {
  const int x = blockIdx.x * 256 + threadIdx.x, J0 = blockIdx.y * 64, bh = blockIdx.z;
  float acc[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) acc[j] = 0.f;
  const uint32_t* km = keep + (size_t)bh * n_kbw * qpad;
  const int w0 = J0 >> 5;
  for (int I = 0; I < n_qb; ++I) {
    const float vx = x < kStateX ? dhm[((size_t)bh * n_qb + I) * kStateX + x] : 0.f;
    const uint32_t m0 = km[(size_t)w0 * qpad + I];
    const uint32_t m1 = (w0 + 1 < n_kbw) ? km[(size_t)(w0 + 1) * qpad + I] : 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if ((m0 >> j) & 1u) acc[j] += vx;
      if ((m1 >> j) & 1u) acc[32 + j] += vx;
    }
  }
  if (x < kStateX)
    for (int j = 0; j < 64; ++j)
      if (J0 + j < n_kb) dhj[((size_t)bh * n_kb + J0 + j) * kStateX + x] = acc[j];
}

// ---------------------------------------------------------------------------------------------------------
// kb_lin_k: grid (n_kb, BH), 256 threads. dphi_k = V dH_J^T + dZ_J; dK += dphi_k * phi'(k); dV += phi(K) dH_J.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kb_lin_k(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                const float* __restrict__ dhj, float* __restrict__ dk,
                                                float* __restrict__ dv, int N, int n_kb) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* sH = (float*)smem;     // [128 c][128 e]
  float* sV = sH + kD * kD;     // [64][128]
  float* sP = sV + 64 * kD;     // [64][128] phi(K)
  float* sZ = sP + 64 * kD;     // [128]
  const int J = blockIdx.x, bh = blockIdx.y, t = threadIdx.x, ty = t >> 4, tx = t & 15;
  const int j0 = J * 64, nk = min(64, N - j0);
  const float* h = dhj + ((size_t)bh * n_kb + J) * kStateX;
  for (int u = t; u < kD * kD; u += 256) sH[u] = h[u];
  for (int u = t; u < kD; u += 256) sZ[u] = h[kD * kD + u];
  const uint16_t* kr = k + ((size_t)bh * N + j0) * kD;
  const uint16_t* vr = v + ((size_t)bh * N + j0) * kD;
  for (int u = t; u < 64 * kD; u += 256) {
    const bool ok = (u >> 7) < nk;
    sV[u] = ok ? bf16_lo(vr[u]) : 0.f;
    sP[u] = ok ? phi_f(bf16_lo(kr[u])) : 0.f;
  }
  __syncthreads();
  VTile<64> dpk, dvl;
  vzero(dpk);
  vzero(dvl);
  vgemm(dpk, sV, kD, 1, sH, 1, kD, kD);  // A[j][e] = V; B[kk = e][col = c] = dH[c][e]
  vgemm(dvl, sP, kD, 1, sH, kD, 1, kD);  // A[j][c] = phi(K); B[kk = c][col = e] = dH[c][e]
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int j = ty + 16 * a;
    if (j < nk)
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int c = tx + 16 * b;
        const size_t o = ((size_t)bh * N + j0 + j) * kD + c;
        dk[o] += (dpk.c[a][b] + sZ[c]) * dphi(bf16_lo(kr[j * kD + c]));
        dv[o] += dvl.c[a][b];
      }
  }
}

// ---------------------------------------------------------------------------------------------------------
// kb_dw: grid (n_chunks, BH), 256 threads: partial [c][e] = sum over the chunk's rows i of O_l[i][c] dY[i][e]
// (rows in ascending order); kb_dw_sum: dW_p = the partials added in (bh, chunk) order.
// ---------------------------------------------------------------------------------------------------------
constexpr int kDwChunk = 1024;

__global__ __launch_bounds__(256) void kb_dw(const float* __restrict__ o_l, const uint16_t* __restrict__ dy,
                                             float* __restrict__ part, int N, int n_chunks) {
  __shared__ float sO[32][kD], sY[32][kD];
  const int ch = blockIdx.x, bh = blockIdx.y, t = threadIdx.x, ty = t >> 4, tx = t & 15;
  const int i0 = ch * kDwChunk, i1 = min(N, i0 + kDwChunk);
  VTile<128> acc;
  vzero(acc);
  for (int s0 = i0; s0 < i1; s0 += 32) {
    const int ns = min(32, i1 - s0);
    __syncthreads();
    for (int u = t; u < 32 * kD; u += 256) {
      const int ii = u >> 7, c = u & 127;
      const bool ok = ii < ns;
      sO[ii][c] = ok ? o_l[((size_t)bh * N + s0 + ii) * kD + c] : 0.f;
      sY[ii][c] = ok ? bf16_lo(dy[((size_t)bh * N + s0 + ii) * kD + c]) : 0.f;
    }
    __syncthreads();
    vgemm(acc, &sO[0][0], 1, kD, &sY[0][0], kD, 1, 32);  // A[row = c][kk = i] = O_l[i][c]; B[kk = i][col = e]
  }
  float* out = part + ((size_t)bh * n_chunks + ch) * kD * kD;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) out[(ty + 16 * a) * kD + tx + 16 * b] = acc.c[a][b];
}

__global__ __launch_bounds__(256) void kb_dw_sum(const float* __restrict__ part, float* __restrict__ dw, int n_parts) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= kD * kD) return;
  float s = 0.f;
  for (int p = 0; p < n_parts; ++p) s += part[(size_t)p * kD * kD + x];
  dw[x] = s;
}

// ---------------------------------------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------------------------------------
size_t kbq_lds_bytes() { return (size_t)(2 * 128 * kLd128 + 2 * 64 * kLd128 + 3 * 128 * kLd64) * 2; }
size_t kbkv_lds_bytes() {
  return (size_t)(2 * 64 * kLd128 + 2 * 128 * kLd64 + 2 * 64 * kLd128 + 4 * 64 * kLd64) * 2 + 2 * 64 * 4;
}
size_t kblinq_lds_bytes() { return (size_t)(2 * kD * kD + 3 * kD + 16 * kD) * 4; }
size_t kblink_lds_bytes() { return (size_t)(kD * kD + 2 * 64 * kD + kD) * 4; }

// dynamic LDS above the default limit is requested once per kernel (gfx950 has 160 KB per workgroup)
template <typename F>
hipError_t allow_lds(F* f, size_t bytes) {
  return hipFuncSetAttribute((const void*)f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_backward_sparse(const BwdPlan& b, hipStream_t s) {
  const Plan& p = *b.fwd;
  hipError_t e0 = allow_lds(kb_q, kbq_lds_bytes());
  if (e0 == hipSuccess) e0 = allow_lds(kb_kv, kbkv_lds_bytes());
  if (e0 != hipSuccess) return e0;
  const int n_qbw = (p.n_qb + 31) / 32;
  hipError_t e = launch_fill_f32((float*)b.sel_bits, (size_t)p.BH * p.n_kb * n_qbw, 0.f, s);
  if (e != hipSuccess) return e;
  if (p.topk > 0) {
    hipLaunchKernelGGL(kb_sel, dim3(p.n_qb, p.BH), dim3(64), 0, s, p.block_idx, b.sel_bits, p.n_qb, p.n_kb, p.topk,
                       n_qbw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kb_q, dim3(p.n_qb, p.BH), dim3(256), kbq_lds_bytes(), s, b.q, b.k, b.v, b.dy, p.block_idx,
                     b.lse, b.dd, b.dq, p.N, p.n_qb, p.n_kb, p.topk, p.blk_q, p.sm_scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kb_kv, dim3(p.n_kb, p.BH), dim3(256), kbkv_lds_bytes(), s, b.q, b.k, b.v, b.dy, b.sel_bits,
                     b.lse, b.dd, b.dk, b.dv, p.N, p.n_qb, p.n_kb, n_qbw, p.blk_q, p.sm_scale);
  return hipGetLastError();
}

hipError_t launch_backward_linear(const BwdPlan& b, hipStream_t s) {
  const Plan& p = *b.fwd;
  hipError_t e0 = allow_lds(kb_lin_q, kblinq_lds_bytes());
  if (e0 == hipSuccess) e0 = allow_lds(kb_lin_k, kblink_lds_bytes());
  if (e0 != hipSuccess) return e0;
  hipLaunchKernelGGL(kb_lin_q, dim3(p.n_qb, p.BH), dim3(256), kblinq_lds_bytes(), s, b.q, b.dy,
                     (const uint16_t*)p.w_proj, p.state_m, b.o_l, b.dq, b.dhm, p.N, p.n_qb, p.blk_q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_kbw = (p.n_kb + 31) / 32, qpad = mask_row_pad(p.n_qb);
  hipLaunchKernelGGL(kb_lin_sum, dim3((kStateX + 255) / 256, (p.n_kb + 63) / 64, p.BH), dim3(256), 0, s, b.dhm,
                     p.keep_mask, b.dhj, p.n_qb, p.n_kb, n_kbw, qpad);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kb_lin_k, dim3(p.n_kb, p.BH), dim3(256), kblink_lds_bytes(), s, b.k, b.v, b.dhj, b.dk, b.dv,
                     p.N, p.n_kb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int n_chunks = (p.N + kDwChunk - 1) / kDwChunk;
  hipLaunchKernelGGL(kb_dw, dim3(n_chunks, p.BH), dim3(256), 0, s, b.o_l, b.dy, b.dw_part, p.N, n_chunks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kb_dw_sum, dim3(kD * kD / 256), dim3(256), 0, s, b.dw_part, b.dw, p.BH * n_chunks);
  return hipGetLastError();
}

size_t backward_dw_chunks(int N) { return (size_t)(N + kDwChunk - 1) / kDwChunk; }

}  // namespace sagesla
