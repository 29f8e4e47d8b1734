// SLA backward for a fixed block selection (gfx950).
//
// "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn) makes SLA trainable (§三(二); the model is
// fine-tuned with it, §四 step 1). The gradient here is that of the float forward for the given selection:
// out = O_s + O_l W_p, O_s the softmax attention over the selected key blocks with scores q.k * sm_scale, O_l the
// elu+1 linear attention over the unselected blocks; INT8 quantization passes straight through and the K-mean
// shift, which leaves every softmax row unchanged, drops out.
//
// Sparse branch (bf16 MFMA, fp32 accumulation; P and dS enter their products rounded to bf16 once, as the
// forward's P does):
//   kb_sel     bitmaps of the selection: [BH][n_kb][ceil(n_qb/32)] (bit I of key block J = I selected J) and
//              [BH][n_qb][ceil(n_kb/32)] (bit J of query block I)
//   kb_q       per query block: pass 1 the log-sum-exp of every row (base 2) and D_i = sum_j P_ij dP_ij, both
//              online; pass 2 dS = P (dP - D) and dQ = dS K sm_scale; writes LSE, D and dQ
//   kb_kv      per key block, over the query blocks that selected it: dV = P^T dY, dK = dS^T Q sm_scale
// Linear branch (bf16 MFMA, hi + lo splits), after the forward's remaining-state product (H_m, Z_m per query block):
//   kb_lin_q   per query block (bf16 MFMA, hi + lo): O_l, dO_l = dY W_p^T, dnum = dO_l / den,
//              dden = -(dO_l . O_l) / den, dQ += (dnum H_m^T + dden Z_m) * phi'(q), and the block's
//              dH_m = phi(Q)^T dnum, dZ_m = phi(Q)^T dden
//   kb_keep_t  the keep mask transposed; dH_J, dZ_J = the sums of dH_m, dZ_m over the query blocks that did not
//              select J, as the forward's dense mask x table product (k4_gemm, bf16 hi + lo MFMA)
//   kb_lin_k   per key block: dK += (V dH_J^T + dZ_J) * phi'(k), dV += phi(K) dH_J (bf16 MFMA, hi + lo)
//   kb_dw      dW_p = sum over all rows of O_l^T dY (bf16 MFMA, O_l as hi + lo; per-chunk partials, then a
//              fixed-order sum in segments)
// With the RMSNorm of Q and K before the path (the attention part then runs at the normalized values):
//   kb_norm_stats, kb_norm_dw, kb_norm_dw_sum, kb_norm_dx carry dq, dk through the norm to the raw inputs and
//   give the gradients of the norm weights
// Every sum has a fixed order; no atomics touch floating-point data.
#include "device_common.h"
#include "internal.h"
#include "lin_common.h"

namespace sagesla {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// accumulator row of register r of a 32x32 MFMA tile (lane l holds column l % 32)
__device__ __forceinline__ int acc_row(int r) { return 8 * (r >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (r & 3); }

typedef __attribute__((address_space(3))) void bw_lds_void;

constexpr int kTileBytes = 64 * 256;  // a swizzled tile: 64 rows of 128 bf16

// (the swizzled tile layout, tswz / toff, and the transposing read are in device_common.h)

// operand of a 32x32x16 MFMA from a swizzled tile: row r0 + l % 32, columns k0 + 8 (l / 32) .. + 7 (l = lane)
__device__ __forceinline__ v8bf row_op(const unsigned char* t, int r0, int k0, int l) {
  return *(const v8bf*)(t + toff(r0 + (l & 31), k0 + 8 * (l >> 5)));
}

// Transposed operand: the MFMA row is tile column m0 + l % 32, and the contraction runs over tile rows i0 .. i0 + 15.
// With AccOrder, slot s (0..7) of lane half g is row i0 + 8 (s / 4) + 4 g + s % 4, the order in which an
// accumulator tile holds its rows, so that a tile of results serves as the other operand where it stands;
// otherwise slot s is row i0 + 8 g + s, the order of an operand read along a row. Two transposing reads: within
// each group of 16 lanes, lane i receives element i % 4 of the 8-byte units addressed by lanes 4 c + i / 4.
template <bool AccOrder = true>
__device__ __forceinline__ v8bf tr_op(const unsigned char* t, int i0, int m0, int l) {
  const int j = l & 15;
  const int r = i0 + (AccOrder ? 4 : 8) * (l >> 5) + (j >> 2);
  const int col = m0 + 16 * ((l >> 4) & 1) + 4 * (j & 3);
  const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + toff(r, col)));
  const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + toff(r + (AccOrder ? 8 : 4), col)));
  const v8s ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(v8bf, ab);
}

// Lane parts of operand addresses in a swizzled tile. Every read is then a lane register plus a compile-time
// offset (tile base, 32-row tile step, 16-row step), with no address arithmetic in the loops.
// row_op(t, r0, 16 s, l) = t + 256 r0 + row_lane_off(l, s) for r0 a multiple of 16
__device__ __forceinline__ uint32_t row_lane_off(int l, int s) {
  const int lr = l & 31, g = l >> 5;
  return (uint32_t)(lr * 256 + 16 * ((2 * s + g) ^ tswz(lr)));
}
// read h of tr_op<true>(t, i0, 32 u, l) = t + 256 i0 + tr_lane_off(l, u, h) for i0 a multiple of 16: the row is
// i0 + 4 g + j / 4 + 8 h, whose tswz is 4 (j / 4) + (g + 2 h) % 4
__device__ __forceinline__ uint32_t tr_lane_off(int l, int u, int h) {
  const int g = l >> 5, j = l & 15, grp = (l >> 4) & 1;
  const int rl = 4 * g + (j >> 2) + 8 * h;
  const int sw = 4 * (j >> 2) + ((g + 2 * h) & 3);
  const int chunk = 4 * u + 2 * grp + ((j & 3) >> 1);
  return (uint32_t)(rl * 256 + 16 * (chunk ^ sw) + 8 * (j & 1));
}
__device__ __forceinline__ v8bf ld_row(const unsigned char* p) { return *(const v8bf*)p; }
__device__ __forceinline__ v8bf ld_tr(const unsigned char* p0, const unsigned char* p1) {
  const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p0);
  const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p1);
  const v8s ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(v8bf, ab);
}

// accumulator rows 8 s .. 8 s + 7 of a lane as one bf16 operand (round to nearest even)
__device__ __forceinline__ v8bf cvt8(const v16f& x, int s) {
  uint32_t h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = pack_bf16x2(x[8 * s + 2 * e], x[8 * s + 2 * e + 1]);
  return __builtin_bit_cast(v8bf, make_uint4(h[0], h[1], h[2], h[3]));
}

// accumulator rows 8 s .. 8 s + 7 of a lane as bf16 hi and lo operands (hi = bf16(x), lo = bf16(x - hi))
__device__ __forceinline__ void split8(const v16f& x, int s, v8bf& hi, v8bf& lo) {
  uint32_t h[4], o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = x[8 * s + 2 * e], b = x[8 * s + 2 * e + 1];
    h[e] = pack_bf16x2(a, b);
    o[e] = pack_bf16x2(a - __uint_as_float(h[e] << 16), b - __uint_as_float(h[e] & 0xffff0000u));
  }
  hi = __builtin_bit_cast(v8bf, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(v8bf, make_uint4(o[0], o[1], o[2], o[3]));
}

__device__ __forceinline__ v16f mfma(v8bf a, v8bf b, v16f c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }

// Wait for this wave's direct-to-LDS loads and LDS accesses, then meet the other waves: the tiles the workgroup
// staged before are complete once every wave passes. The empty asm statements keep LDS accesses on their side.
__device__ __forceinline__ void dma_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0), lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for this wave's LDS accesses only, then meet the other waves: every wave is done with the tiles it read
// (vector-memory loads in flight are left running; a __syncthreads would wait for them too).
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 (no wait), expcnt 7, lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct-to-LDS staging of one 64-row tile of a [rows][128] bf16 matrix: wave w issues four loads of 1 KB (tile
// rows 16 e + 4 w .. + 3); lane l fills row 16 e + 4 w + l / 16 at chunk position l % 16 with the chunk
// (l % 16) ^ tswz(row). Tile rows at or past nvalid re-read the last valid row (finite values that the kernels
// weight by zero), so no load leaves the matrix.
struct TileLoader {
  int row[4];
  uint32_t chunk[4];
  __device__ __forceinline__ TileLoader() {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      row[e] = 16 * e + 4 * w + (l >> 4);
      chunk[e] = (uint32_t)(16 * ((l & 15) ^ tswz(row[e])));
    }
  }
  __device__ __forceinline__ void operator()(__amdgpu_buffer_rsrc_t src, int row0, int nvalid, unsigned char* tile) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t off = (uint32_t)(row0 + min(row[e], nvalid - 1)) * 256u + chunk[e];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (bw_lds_void*)(tile + (4 * e + w) * 1024), 16, off, 0, 0, 0);
    }
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int N) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, N * kD * 2, 0x00020000);
}

}  // namespace

// ---------------------------------------------------------------------------------------------------------
// kb_sel: grid (n_qb, BH), 64 threads. Sets bit I of word [bh][J][I / 32] and bit J of word [bh][I][J / 32] for
// every listed J (atomic OR: the result does not depend on the order; a block listed twice sets its bits once).
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void kb_sel(const int32_t* __restrict__ idx, uint32_t* __restrict__ bits,
                                             uint32_t* __restrict__ bits_q, int n_qb, int n_kb, int topk, int n_qbw,
                                             int n_kbw) {
  const int I = blockIdx.x, bh = blockIdx.y;
  const int32_t* row = idx + ((size_t)bh * n_qb + I) * topk;
  for (int t = threadIdx.x; t < topk; t += 64) {
    const int J = min(max(row[t], 0), n_kb - 1);
    atomicOr(&bits[((size_t)bh * n_kb + J) * n_qbw + (I >> 5)], 1u << (I & 31));
    atomicOr(&bits_q[((size_t)bh * n_qb + I) * n_kbw + (J >> 5)], 1u << (J & 31));
  }
}

// ---------------------------------------------------------------------------------------------------------
// kb_q: grid (n_qb, BH), 256 threads (4 waves x 32 query rows), two workgroups per CU. Scores are computed
// transposed, S^T = K Q^T, so each lane owns one query row (with its partner lane l ^ 32); the wave's Q and dY
// rows stay in registers as the B operands. The selected key blocks (ascending, each once, from the bitmap)
// stream through a two-slot ring of swizzled K and V tiles filled by direct-to-LDS loads one block ahead.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void kb_q(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                               const uint16_t* __restrict__ v, const uint16_t* __restrict__ dy,
                                               const uint32_t* __restrict__ bits_q, float* __restrict__ lse_out,
                                               float* __restrict__ d_out, float* __restrict__ dq, int N, int n_qb,
                                               int n_kbw, int blk_q, float sm_scale) {
  extern __shared__ __align__(1024) unsigned char smem[];  // [slot][K tile, V tile]
  const int I = blockIdx.x, bh = blockIdx.y;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63, g = l >> 5;
  const int r0 = I * blk_q, nq = min(blk_q, N - r0);
  const bool wave_live = 32 * w < nq;  // blk_q 64: waves 2, 3 hold no rows but still stage and meet
  const int i_loc = 32 * w + (l & 31);
  const float c2 = sm_scale * kLog2e;
  v8bf qb[8], yb[8];
  {
    const bool iv = i_loc < nq;
    const uint16_t* qr = q + ((size_t)bh * N + r0 + (iv ? i_loc : 0)) * kD + 8 * g;
    const uint16_t* yr = dy + ((size_t)bh * N + r0 + (iv ? i_loc : 0)) * kD + 8 * g;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qb[s] = iv ? *(const v8bf*)(qr + 16 * s) : (v8bf){};
      yb[s] = iv ? *(const v8bf*)(yr + 16 * s) : (v8bf){};
    }
  }
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(k + (size_t)bh * N * kD, N);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(v + (size_t)bh * N * kD, N);
  const TileLoader load;
  const uint32_t* sb = bits_q + ((size_t)bh * n_qb + I) * n_kbw;
  // lane parts of the tile addresses, opaque so that the compiler keeps these 16 registers rather than
  // materializing one address per read
  uint32_t ro[8], to[4][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    ro[s] = row_lane_off(l, s);
    asm volatile("" : "+v"(ro[s]));
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      to[u][h] = tr_lane_off(l, u, h);
      asm volatile("" : "+v"(to[u][h]));
    }
  // the selected blocks in ascending order: a cursor over the bitmap words (uniform across the workgroup)
  auto next_block = [&](int& wi, uint32_t& cw) -> int {
    while (cw == 0) {
      if (++wi >= n_kbw) return -1;
      cw = sb[wi];
    }
    const int J = 32 * wi + __builtin_ctz(cw);
    cw &= cw - 1;
    return J;
  };
  auto stage = [&](int J, int slot) {
    unsigned char* t = smem + slot * 2 * kTileBytes;
    const int nv = min(64, N - J * 64);
    load(rk, J * 64, nv, t);
    load(rv, J * 64, nv, t + kTileBytes);
  };
  // Runs body(J, K tile, V tile) over the selected blocks through the two-slot ring; the loop is unrolled by two
  // so that each slot's tile addresses are constants.
  auto ring = [&](auto&& body) {
    auto run = [&](int J, const unsigned char* tk, const unsigned char* tv) {
      if (wave_live) body(J, tk, tv);
    };
    int wi = 0;
    uint32_t cw = sb[0];
    int cur = next_block(wi, cw);
    if (cur >= 0) stage(cur, 0);
    while (cur >= 0) {
      int nxt = next_block(wi, cw);
      dma_sync();
      if (nxt >= 0) stage(nxt, 1);
      run(cur, smem, smem + kTileBytes);
      cur = nxt;
      if (cur < 0) break;
      nxt = next_block(wi, cw);
      dma_sync();
      if (nxt >= 0) stage(nxt, 0);
      run(cur, smem + 2 * kTileBytes, smem + 3 * kTileBytes);
      cur = nxt;
    }
  };
  // Only the head's last key block can hold fewer than 64 keys: there (a uniform branch) the scores of keys past
  // N (rows re-read from the last valid key) are set to -inf, so that their exp2 is 0
  const int ragged_J = (N % 64) ? (N - 1) / 64 : -1;
  auto mask_tail = [&](v16f& st, int tt, int J) {
    if (J != ragged_J) return;
    const int nv = N - J * 64;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * tt + acc_row(r) >= nv) st[r] = -INFINITY;
  };
  // S^T and dP^T of one 32-key tile tt of the block in tiles tk (K), tv (V)
  auto tile_sdp = [&](const unsigned char* tk, const unsigned char* tv, int tt, v16f& st, v16f& dp) {
    st = (v16f){};
    dp = (v16f){};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      st = mfma(ld_row(tk + 8192 * tt + ro[s]), qb[s], st);
      dp = mfma(ld_row(tv + 8192 * tt + ro[s]), yb[s], dp);
    }
  };

  // pass 1, online per row: m = max of s * c2, l = sum of 2^(s c2 - m) and u = sum of 2^(s c2 - m) dP, both
  // rescaled when m grows; then LSE = m + log2(l) and D = u / l = sum_j P_ij dP_ij
  float m = -INFINITY, lsum = 0.f, usum = 0.f;
  ring([&](int J, const unsigned char* tk, const unsigned char* tv) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      v16f st, dp;
      tile_sdp(tk, tv, tt, st, dp);
      mask_tail(st, tt, J);
      // the tile's largest score times c2 > 0 (tile 0 always holds a valid key, so m is finite after it)
      float bm = st[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) bm = fmaxf(bm, st[r]);
      bm = fmaxf(bm, swap_halves_f32(bm)) * c2;
      const float mn = fmaxf(m, bm);
      float ps = 0.f, pu = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ev = __builtin_amdgcn_exp2f(fmaf(st[r], c2, -mn));
        ps += ev;
        pu = fmaf(ev, dp[r], pu);
      }
      ps += swap_halves_f32(ps);
      pu += swap_halves_f32(pu);
      const float sc = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
      lsum = lsum * sc + ps;
      usum = usum * sc + pu;
      m = mn;
    }
  });
  const float lse = (lsum > 0.f) ? m + __log2f(lsum) : 0.f;  // no selected key: every P is 0 below
  const float dsum = (lsum > 0.f) ? usum / lsum : 0.f;
  if (wave_live && l < 32 && i_loc < nq) {
    lse_out[(size_t)bh * N + r0 + i_loc] = lse;
    d_out[(size_t)bh * N + r0 + i_loc] = dsum;
  }

  // pass 2: dS^T = P (dP - D) per tile in registers, dQ^T += K^T dS^T with K^T read transposed from the K tile
  v16f acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = (v16f){};
  __syncthreads();  // pass 1's reads of both slots are done
  ring([&](int J, const unsigned char* tk, const unsigned char* tv) {
    const float nl2 = -lse;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      v16f st, dp;
      tile_sdp(tk, tv, tt, st, dp);
      mask_tail(st, tt, J);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[r], c2, nl2));
        st[r] = p * (dp[r] - dsum);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const v8bf ds = cvt8(st, s);
        const unsigned char* rb = tk + 8192 * tt + 4096 * s;
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = mfma(ld_tr(rb + to[u][0], rb + to[u][1]), ds, acc[u]);
      }
    }
  });
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
// kb_kv: grid (n_kb, BH), 256 threads, two workgroups per CU: wave w takes keys 32 (w % 2) .. +31 and rows
// 32 (w / 2) .. +31 of each 64-row half of a query block. K and V of the block are staged once; for every query
// block I that selected J (bitmap) the halves of Q and dY are staged as swizzled tiles, S = Q K^T and
// dP = dY V^T are formed with the keys as columns (lane = key), and P and dS, still in their accumulator
// registers, are the B operands of dV^T += dY^T P and dK^T += Q^T dS, whose A operands are read transposed
// from the Q and dY tiles. The two waves of a key tile then hold partial sums over complementary rows, added in a
// fixed order at the end.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void kb_kv(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                const uint16_t* __restrict__ v, const uint16_t* __restrict__ dy,
                                                const uint32_t* __restrict__ bits, const float* __restrict__ lse_in,
                                                const float* __restrict__ d_in, float* __restrict__ dk,
                                                float* __restrict__ dv, int N, int n_kb, int n_qbw, int blk_q,
                                                float sm_scale) {
  extern __shared__ __align__(1024) unsigned char smem[];
  unsigned char* sK = smem;
  unsigned char* sV = smem + kTileBytes;
  unsigned char* sQ = smem + 2 * kTileBytes;
  unsigned char* sdY = smem + 3 * kTileBytes;
  float* sL = (float*)(smem + 4 * kTileBytes);  // [64] LSE of the half's rows
  float* sDd = sL + 64;                          // [64] D of the half's rows
  const int J = blockIdx.x, bh = blockIdx.y;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int kt = w & 1, ch = w >> 1;  // key tile, row chunk
  const int nk = min(64, N - J * 64);
  const float c2 = sm_scale * kLog2e;
  const TileLoader load;
  const __amdgpu_buffer_rsrc_t rq = head_rsrc(q + (size_t)bh * N * kD, N);
  const __amdgpu_buffer_rsrc_t ry = head_rsrc(dy + (size_t)bh * N * kD, N);
  load(head_rsrc(k + (size_t)bh * N * kD, N), J * 64, nk, sK);
  load(head_rsrc(v + (size_t)bh * N * kD, N), J * 64, nk, sV);
  const int j_loc = 32 * kt + (l & 31);
  // lane parts of the tile addresses (the wave's row chunk folded in), kept opaque so that the compiler holds
  // three registers rather than one address per read. Row reads of k-step sd use the lane part of step 0 with
  // bits 5-7 flipped by sd; the transposed reads of column tile u the lane part of tile 0 with bits 6-7 flipped
  // by u (no other bit of a lane part reaches those bits). The K and V rows of the wave's key tile are the Q and
  // dY lane parts shifted by the wave-uniform 8192 (kt - ch).
  uint32_t oq = row_lane_off(l, 0) + 8192u * ch, tq[2];
  asm volatile("" : "+v"(oq));
  const int dkv = 8192 * (kt - ch);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    tq[h] = tr_lane_off(l, 0, h) + 8192u * ch;
    asm volatile("" : "+v"(tq[h]));
  }
  v16f accv[4], acck[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) accv[u] = acck[u] = (v16f){};
  // the steps: (query block I that selected J, 64-row half h0), in order; a cursor over the bitmap words (read
  // through the constant address space: scalar loads, which leave the vector-memory counter to the tile loads)
  typedef __attribute__((address_space(4))) const uint32_t c_u32;
  c_u32* jb = (c_u32*)(bits + ((size_t)bh * n_kb + J) * n_qbw);
  int wd = 0;
  uint32_t word = jb[0];
  auto next_I = [&]() -> int {
    while (word == 0) {
      if (++wd >= n_qbw) return -1;
      word = jb[wd];
    }
    const int I = 32 * wd + __builtin_ctz(word);
    word &= word - 1;
    return I;
  };
  int I = next_I(), h0 = 0;
  while (I >= 0) {
    {
      const int q0 = I * blk_q, nq = min(blk_q, N - q0);
      const int nh = min(64, nq - h0);
      int In = I, hn = h0 + 64;
      if (hn >= nq) {
        In = next_I();
        hn = 0;
      }
      lds_sync();  // the previous half's tiles are no longer read
      // the half's row statistics are loaded before its tiles, so that storing them waits for them alone
      float lse_r = 0.f, d_r = 0.f;
      if (threadIdx.x < nh) {
        lse_r = lse_in[(size_t)bh * N + q0 + h0 + threadIdx.x];
        d_r = d_in[(size_t)bh * N + q0 + h0 + threadIdx.x];
      }
      load(rq, q0 + h0, nh, sQ);
      load(ry, q0 + h0, nh, sdY);
      if (threadIdx.x < 64) {
        sL[threadIdx.x] = lse_r;
        sDd[threadIdx.x] = d_r;
      }
      dma_sync();
      I = In;
      h0 = hn;
      v16f s = (v16f){}, dp = (v16f){};
#pragma unroll
      for (int sd = 0; sd < 8; ++sd) {
        const uint32_t o = oq ^ (32u * sd), okv = o + dkv;
        s = mfma(ld_row(sQ + o), ld_row(sK + okv), s);
        dp = mfma(ld_row(sdY + o), ld_row(sV + okv), dp);
      }
      // s[r] -> P, dp[r] -> dS for row 32 ch + acc_row(r) and key j_loc (the fences keep the row statistics'
      // reads and the transposed operand reads from being hoisted while every accumulator is live)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ii = 32 * ch + acc_row(r);  // < 64: the row statistics are read unconditionally
        const float e = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -sL[ii]));
        const float p = ii < nh ? e : 0.f;
        dp[r] = p * (dp[r] - sDd[ii]);
        s[r] = p;
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        __builtin_amdgcn_sched_barrier(0);
        const v8bf pb = cvt8(s, st), db = cvt8(dp, st);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t t0 = tq[0] ^ (64u * u), t1 = tq[1] ^ (64u * u);
          accv[u] = mfma(ld_tr(sdY + 4096 * st + t0, sdY + 4096 * st + t1), pb, accv[u]);
          acck[u] = mfma(ld_tr(sQ + 4096 * st + t0, sQ + 4096 * st + t1), db, acck[u]);
        }
      }
    }
  }
  // acc[u][r] = partial X^T[d = 32 u + acc_row(r)][key j_loc] over the rows of chunk ch: chunk 1 hands its sums
  // to chunk 0 through LDS (the tiles are free now, and the K and V loads have landed even when no query block
  // selected J), which adds them (chunk 0 first) and stores
  dma_sync();
  float* sX = (float*)smem;  // [2 key tiles][2 (dV, dK)][4 u][16 r][64 lanes] = 64 KB
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

__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : __builtin_amdgcn_exp2f(x * kLog2e); }

// ---------------------------------------------------------------------------------------------------------
// kb_lin_q: grid (n_qb, BH), 256 threads (4 waves); bf16 MFMA with hi + lo splits of every non-bf16 operand.
// For query block I with its remaining state H_m (record planes of H_m^T, row e) and Z_m:
//   num = phi(Q) H_m, den = phi(Q) . Z_m, O_l = num / den (stored for dW_p)
//   dO_l = dY W_p^T, dnum = dO_l / den
//   dH_m = phi(Q)^T dnum                                    (wave w: columns e of tile w, contraction over rows)
//   G = dnum H_m^T, dden = -(phi(Q) . G) / den              (= -(dO_l . O_l) / den; wave w: rows i of tile w)
//   dQ += (G + dden Z_m) phi'(Q), dZ_m = phi(Q)^T dden
// LDS: phi(Q) as hi + lo tiles (later dnum^T), the planes of H_m^T as hi + lo tiles.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kb_lin_q(const uint16_t* __restrict__ q, const uint16_t* __restrict__ dy,
                                                const uint16_t* __restrict__ w_proj, const float* __restrict__ state_m,
                                                float* __restrict__ o_l, float* __restrict__ dq,
                                                float* __restrict__ dhm, int N, int n_qb, int blk_q) {
  extern __shared__ __align__(1024) unsigned char smem[];
  unsigned char* sPh = smem;                    // 128-row tiles: phi(Q) [i][c] hi, lo; later dnum^T [e][i]
  unsigned char* sPl = smem + 2 * kTileBytes;
  unsigned char* sHh = smem + 4 * kTileBytes;   // H_m^T [e][c] hi, lo
  unsigned char* sHl = smem + 6 * kTileBytes;
  float* sZ = (float*)(smem + 8 * kTileBytes);  // [128]
  float* sInv = sZ + kD;                        // [128] 1 / den (0 past nq)
  float* sDd = sInv + kD;                       // [128] dden
  const int I = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, g = l >> 5;
  const int r0 = I * blk_q, nq = min(blk_q, N - r0);
  const unsigned char* rec = (const unsigned char*)state_m + ((size_t)bh * n_qb + I) * (size_t)kStateX * 4;
  const uint16_t* qr = q + ((size_t)bh * N + r0) * kD;
  const uint16_t* dyr = dy + ((size_t)bh * N + r0) * kD;
  const float* zg = (const float*)(rec + 65536);

  // staging: thread t takes row i = t / 2, columns 64 (t % 2) .. +63 of phi(Q) (zero past nq) and its part of
  // den[i]; the two halves are added through the neighbouring lane (fixed order)
  {
    const int i = t >> 1, hc = t & 1;
    float dpart = 0.f;
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) {
      const int c0 = 64 * hc + 8 * qq;
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (i < nq) raw = *(const uint4*)(qr + i * kD + c0);
      const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
      const float4 z0 = *(const float4*)(zg + c0), z1 = *(const float4*)(zg + c0 + 4);
      const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
      uint32_t h[4], o[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float x0 = i < nq ? phi_f(bf16_lo(wv[e2])) : 0.f, x1 = i < nq ? phi_f(bf16_lo(wv[e2] >> 16)) : 0.f;
        dpart = fmaf(x0, zz[2 * e2], dpart);
        dpart = fmaf(x1, zz[2 * e2 + 1], dpart);
        h[e2] = pack_bf16x2(x0, x1);
        o[e2] = pack_bf16x2(x0 - __uint_as_float(h[e2] << 16), x1 - __uint_as_float(h[e2] & 0xffff0000u));
      }
      *(uint4*)(sPh + toff(i, c0)) = make_uint4(h[0], h[1], h[2], h[3]);
      *(uint4*)(sPl + toff(i, c0)) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    const float other = __shfl_xor(dpart, 1);
    if (hc == 0) sInv[i] = i < nq ? 1.f / (dpart + other) : 0.f;  // the divisions below become products
  }
#pragma unroll
  for (int it = 0; it < 16; ++it) {  // the planes of H_m^T, re-swizzled: 2 planes x 128 rows x 16 chunks
    const int u = t + 256 * it, pl = u >> 11, e = (u >> 4) & 127, qq = u & 15;
    const uint4 x = *(const uint4*)(rec + 32768 * pl + out_off(e, 8 * qq));
    *(uint4*)((pl ? sHl : sHh) + toff(e, 8 * qq)) = x;
  }
  if (t < kD) sZ[t] = zg[t];
  __syncthreads();

  // num (wave w: columns e of tile w, all rows): D[i][e] = sum_c phi(Q)[i][c] H_m[c][e]
  const int ecol = 32 * w + (l & 31);
  v16f acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = (v16f){};
#pragma unroll 2
  for (int s = 0; s < 8; ++s) {
    const v8bf bh_ = row_op(sHh, 32 * w, 16 * s, l), bl_ = row_op(sHl, 32 * w, 16 * s, l);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const v8bf ah = row_op(sPh, 32 * a, 16 * s, l), al = row_op(sPl, 32 * a, 16 * s, l);
      acc[a] = mfma(ah, bh_, acc[a]);
      acc[a] = mfma(ah, bl_, acc[a]);
      acc[a] = mfma(al, bh_, acc[a]);
    }
  }
  // O_l = num / den, stored for dW_p
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * a + acc_row(r);
      if (i < nq) o_l[((size_t)bh * N + r0 + i) * kD + ecol] = acc[a][r] * sInv[i];
    }

  // dO_l (same tiles): D[i][e] = sum_f dY[i][f] W_p[e][f]; A read from global rows of dY, B from rows of W_p
  v8bf wb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) wb[s] = *(const v8bf*)(w_proj + (size_t)ecol * kD + 16 * s + 8 * g);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    acc[a] = (v16f){};
    const int i = 32 * a + (l & 31);
    const uint16_t* yrow = dyr + (size_t)min(i, nq - 1) * kD + 8 * g;
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[a] = mfma(*(const v8bf*)(yrow + 16 * s), wb[s], acc[a]);
  }
  // dnum = dO_l / den (0 on rows past nq, whose 1 / den is stored as 0)
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[a][r] *= sInv[32 * a + acc_row(r)];

  // dH_m (wave w: columns e of tile w): D[c][e] = sum_i phi(Q)^T[c][i] dnum[i][e], phi(Q)^T read transposed in
  // accumulator row order so that dnum serves as B from its registers
  {
    v16f dh[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) dh[ct] = (v16f){};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      v8bf nh, nl;
      split8(acc[s >> 1], s & 1, nh, nl);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const v8bf ah = tr_op(sPh, 16 * s, 32 * ct, l), al = tr_op(sPl, 16 * s, 32 * ct, l);
        dh[ct] = mfma(ah, nh, dh[ct]);
        dh[ct] = mfma(ah, nl, dh[ct]);
        dh[ct] = mfma(al, nh, dh[ct]);
      }
    }
    // column-tiled table: dH_m[c][e] at column group c, column e
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * ct + acc_row(r);
        dhm[(((size_t)bh * (kStateX / 128) + c) * n_qb + I) * 128 + ecol] = dh[ct][r];
      }
  }
  __syncthreads();  // phi(Q) tiles no longer read
  // dnum^T [e][i] as hi + lo into the phi(Q) tiles: lane e, runs of four rows i -> 8-byte pieces
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      const int i0 = 32 * a + acc_row(r);
      uint32_t h0 = pack_bf16x2(acc[a][r], acc[a][r + 1]), h1 = pack_bf16x2(acc[a][r + 2], acc[a][r + 3]);
      uint32_t o0 = pack_bf16x2(acc[a][r] - __uint_as_float(h0 << 16), acc[a][r + 1] - __uint_as_float(h0 & 0xffff0000u));
      uint32_t o1 = pack_bf16x2(acc[a][r + 2] - __uint_as_float(h1 << 16), acc[a][r + 3] - __uint_as_float(h1 & 0xffff0000u));
      *(uint2*)(sPh + toff(ecol, i0)) = make_uint2(h0, h1);
      *(uint2*)(sPl + toff(ecol, i0)) = make_uint2(o0, o1);
    }
  __syncthreads();

  // G (wave w: rows i of tile w, all columns c): D[c][i] = sum_e H_m[c][e] dnum[i][e], both operands read
  // transposed (contraction over the rows e of the H_m^T and dnum^T tiles)
  const int irow = 32 * w + (l & 31);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = (v16f){};
#pragma unroll 2
  for (int s = 0; s < 8; ++s) {
    const v8bf bh_ = tr_op<false>(sPh, 16 * s, 32 * w, l), bl_ = tr_op<false>(sPl, 16 * s, 32 * w, l);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const v8bf ah = tr_op<false>(sHh, 16 * s, 32 * ct, l), al = tr_op<false>(sHl, 16 * s, 32 * ct, l);
      acc[ct] = mfma(ah, bh_, acc[ct]);
      acc[ct] = mfma(ah, bl_, acc[ct]);
      acc[ct] = mfma(al, bh_, acc[ct]);
    }
  }
  // dden[i] = -(phi(Q)[i] . G[i]) / den[i]; lane i holds c = 32 ct + acc_row(r), the partner lane the rest
  const bool iv = irow < nq;
  const uint16_t* qrow = qr + (size_t)(iv ? irow : 0) * kD;
  float dot = 0.f;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      const uint2 raw = iv ? *(const uint2*)(qrow + 32 * ct + acc_row(r)) : make_uint2(0, 0);
      const uint32_t wv[2] = {raw.x, raw.y};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float x = bf16_lo(e2 & 1 ? wv[e2 >> 1] >> 16 : wv[e2 >> 1]);
        dot = fmaf(iv ? phi_f(x) : 0.f, acc[ct][r + e2], dot);
      }
    }
  dot += swap_halves_f32(dot);
  const float dden = iv ? -dot * sInv[irow] : 0.f;
  if (l < 32) sDd[irow] = dden;
  if (iv) {
    // read-modify-write of dQ: every load (dQ and the q values) issued before the first store
    float* dst = dq + ((size_t)bh * N + r0 + irow) * kD;
    float4 dold[16];
    uint2 qraw[16];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int c0 = 32 * ct + acc_row(r);
        dold[4 * ct + r / 4] = *(const float4*)(dst + c0);
        qraw[4 * ct + r / 4] = *(const uint2*)(qrow + c0);
      }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int c0 = 32 * ct + acc_row(r);
        const uint32_t wv[2] = {qraw[4 * ct + r / 4].x, qraw[4 * ct + r / 4].y};
        float4 d = dold[4 * ct + r / 4];
        float* dd = (float*)&d;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float x = bf16_lo(e2 & 1 ? wv[e2 >> 1] >> 16 : wv[e2 >> 1]);
          dd[e2] += (acc[ct][r + e2] + dden * sZ[c0 + e2]) * dphi(x);
        }
        *(float4*)(dst + c0) = d;
      }
  }
  __syncthreads();  // G's reads of the H_m^T tiles are done and dden is in LDS
  // dZ_m[c] = sum_i phi(Q)[i][c] dden[i]: the block's Q rows into the free H_m^T tile (all loads issued before
  // any is waited for), then per column two half sums (rows 0-63 and 64-127, ascending) added in that order
  {
    uint4 x[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int u = t + 256 * it, i = u >> 4;
      x[it] = i < nq ? *(const uint4*)(qr + (size_t)i * kD + 8 * (u & 15)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int u = t + 256 * it;
      *(uint4*)(sHh + 16 * u) = x[it];  // row u / 16 at 256 (u / 16), unswizzled
    }
  }
  __syncthreads();
  {
    const int c = t & 127, half = t >> 7;
    const uint16_t* qs = (const uint16_t*)sHh;
    float sz = 0.f;
#pragma unroll 8
    for (int i = 64 * half; i < 64 * half + 64; ++i)
      if (i < nq) sz = fmaf(phi_f(bf16_lo(qs[i * kD + c])), sDd[i], sz);
    float* part = (float*)sHl;
    if (half == 1) part[c] = sz;
    __syncthreads();
    if (half == 0) dhm[(((size_t)bh * (kStateX / 128) + kD) * n_qb + I) * 128 + c] = sz + part[c];
  }
}

// ---------------------------------------------------------------------------------------------------------
// kb_keep_t: the keep mask transposed for the sum over query blocks, keep_t[bh][w][J] (rows padded to kpad):
// bit i = 1 iff query block 32 w + i exists and did not select key block J (the complement of the selection
// bitmap); padding rows are 0. The sums dH_J = sum over those query blocks of dH_m then run as the same dense
// mask x table product as the forward's remaining states.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kb_keep_t(const uint32_t* __restrict__ sel_bits, uint32_t* __restrict__ keep_t,
                                                 int n_qb, int n_kb, int n_qbw, int kpad, size_t total) {
  const size_t x = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= total) return;
  const int J = (int)(x % kpad);
  const size_t r = x / kpad;
  const int w = (int)(r % n_qbw), bh = (int)(r / n_qbw);
  uint32_t v = 0u;
  if (J < n_kb) {
    const int left = n_qb - 32 * w;
    const uint32_t valid = left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
    v = ~sel_bits[((size_t)bh * n_kb + J) * n_qbw + w] & valid;
  }
  keep_t[x] = v;
}

// ---------------------------------------------------------------------------------------------------------
// kb_lin_k: grid (n_kb, BH), 512 threads (8 waves). For key block J with its dH_J (the record's bf16 hi + lo
// planes, row c) and dZ_J:
//   dphi_k[j][c] = sum_e V[j][e] dH[c][e] + dZ[c];  dK[j][c] += dphi_k[j][c] phi'(K[j][c])
//   dV[j][e] += sum_c phi(K)[j][c] dH[c][e]
// on bf16 MFMA: V is exact, dH enters as hi + lo, phi(K) is split into hi + lo in registers (three products,
// hi.hi + hi.lo + lo.hi). The planes are re-swizzled into LDS; K and V arrive by direct-to-LDS loads. Wave w owns
// key tile w / 4 and column tile w % 4 (c for dK, e for dV).
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(512) void kb_lin_k(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                const float* __restrict__ dhj, float* __restrict__ dk,
                                                float* __restrict__ dv, int N, int n_kb) {
  extern __shared__ __align__(1024) unsigned char smem[];
  unsigned char* sK = smem;                      // 64-row tiles
  unsigned char* sV = smem + kTileBytes;
  unsigned char* sHh = smem + 2 * kTileBytes;    // 128-row tiles: dH hi, lo (row c, column e)
  unsigned char* sHl = sHh + 2 * kTileBytes;
  float* sZ = (float*)(sHl + 2 * kTileBytes);    // [128]
  const int J = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int jt = w >> 2, ct = w & 3;
  const int j0 = J * 64, nk = min(64, N - j0);
  if (w < 4) {  // the loader's wave layout covers 4 waves
    const TileLoader load;
    load(head_rsrc(k + (size_t)bh * N * kD, N), j0, nk, sK);
    load(head_rsrc(v + (size_t)bh * N * kD, N), j0, nk, sV);
  }
  const unsigned char* rec = (const unsigned char*)(dhj + ((size_t)bh * n_kb + J) * kStateX);
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // 2 planes x 128 rows x 16 chunks
    const int u = t + 512 * i, pl = u >> 11, c = (u >> 4) & 127, q = u & 15;
    const uint4 x = *(const uint4*)(rec + 32768 * pl + out_off(c, 8 * q));
    *(uint4*)((pl ? sHl : sHh) + toff(c, 8 * q)) = x;
  }
  if (t < kD) sZ[t] = *(const float*)(rec + 65536 + 4 * t);
  dma_sync();
  v16f acck = (v16f){}, accv = (v16f){};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    // dphi_k^T... as D[j][c]: A = V rows j (k = e), B = dH rows c (k = e)
    const v8bf av = row_op(sV, 32 * jt, 16 * s, l);
    acck = mfma(av, row_op(sHh, 32 * ct, 16 * s, l), acck);
    acck = mfma(av, row_op(sHl, 32 * ct, 16 * s, l), acck);
    // dV as D[j][e]: A = phi(K) rows j (k = c) as hi + lo, B = dH^T (column e, k = c) read transposed
    const v8bf kr = row_op(sK, 32 * jt, 16 * s, l);
    uint32_t ph[4], plo[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const uint32_t wv = __builtin_bit_cast(uint4, kr)[e2];
      const float x0 = phi_f(bf16_lo(wv)), x1 = phi_f(bf16_lo(wv >> 16));
      ph[e2] = pack_bf16x2(x0, x1);
      plo[e2] = pack_bf16x2(x0 - __uint_as_float(ph[e2] << 16), x1 - __uint_as_float(ph[e2] & 0xffff0000u));
    }
    const v8bf ah = __builtin_bit_cast(v8bf, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const v8bf al = __builtin_bit_cast(v8bf, make_uint4(plo[0], plo[1], plo[2], plo[3]));
    const v8bf bh_ = tr_op<false>(sHh, 16 * s, 32 * ct, l);
    const v8bf bl_ = tr_op<false>(sHl, 16 * s, 32 * ct, l);
    accv = mfma(ah, bh_, accv);
    accv = mfma(ah, bl_, accv);
    accv = mfma(al, bh_, accv);
  }
  // acc[r]: key j = 32 jt + acc_row(r), column 32 ct + l % 32 (c for dK, e for dV)
  const int col = 32 * ct + (l & 31);
  const float zc = sZ[col];
  // read-modify-write of dK and dV: every load issued before the first store (a store between them would make
  // each load wait for the previous one)
  float okv[16], ovv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = 32 * jt + acc_row(r);
    const size_t o = ((size_t)bh * N + j0 + min(j, nk - 1)) * kD + col;
    okv[r] = dk[o];
    ovv[r] = dv[o];
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = 32 * jt + acc_row(r);
    if (j < nk) {
      const size_t o = ((size_t)bh * N + j0 + j) * kD + col;
      const float kv = bf16_lo(*(const uint16_t*)(sK + toff(j, col & ~3) + 2 * (col & 3)));
      dk[o] = okv[r] + (acck[r] + zc) * dphi(kv);
      dv[o] = ovv[r] + accv[r];
    }
  }
}

// ---------------------------------------------------------------------------------------------------------
// kb_dw: grid (n_chunks, BH), 256 threads (4 waves): partial [e][f] = sum over the chunk's rows i of
// O_l[i][e] dY[i][f] on bf16 MFMA, O_l as hi + lo. Steps of 64 rows: O_l (hi, lo) and dY are staged as swizzled
// tiles; A = O_l^T and B = dY^T come from transposing reads (contraction over the rows, in row order). Wave w
// owns output rows e of tile w and all columns f. kb_dw_sum1 / kb_dw_sum2: dW_p = the partials added in
// (bh, chunk) order, in kDwSeg segments and then over the segments.
// ---------------------------------------------------------------------------------------------------------
constexpr int kDwChunk = 1024;
constexpr int kDwSeg = 64;

__global__ __launch_bounds__(256) void kb_dw(const float* __restrict__ o_l, const uint16_t* __restrict__ dy,
                                             float* __restrict__ part, int N, int n_chunks) {
  __shared__ __align__(1024) unsigned char sOh[kTileBytes], sOl[kTileBytes], sY[kTileBytes];
  const int ch = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int i0 = ch * kDwChunk, i1 = min(N, i0 + kDwChunk);
  v16f acc[4];
#pragma unroll
  for (int ft = 0; ft < 4; ++ft) acc[ft] = (v16f){};
  for (int s0 = i0; s0 < i1; s0 += 64) {
    const int ns = min(64, i1 - s0);
    __syncthreads();  // the previous step's tiles are no longer read
#pragma unroll
    for (int it = 0; it < 8; ++it) {  // O_l: 64 rows x 32 groups of 4 columns
      const int u = t + 256 * it, row = u >> 5, c4 = 4 * (u & 31);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row < ns) x = *(const float4*)(o_l + ((size_t)bh * N + s0 + row) * kD + c4);
      const uint32_t h0 = pack_bf16x2(x.x, x.y), h1 = pack_bf16x2(x.z, x.w);
      const uint32_t q0 = pack_bf16x2(x.x - __uint_as_float(h0 << 16), x.y - __uint_as_float(h0 & 0xffff0000u));
      const uint32_t q1 = pack_bf16x2(x.z - __uint_as_float(h1 << 16), x.w - __uint_as_float(h1 & 0xffff0000u));
      *(uint2*)(sOh + toff(row, c4)) = make_uint2(h0, h1);
      *(uint2*)(sOl + toff(row, c4)) = make_uint2(q0, q1);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {  // dY: 64 rows x 16 chunks of 8 columns
      const int u = t + 256 * it, row = u >> 4, c8 = 8 * (u & 15);
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row < ns) x = *(const uint4*)(dy + ((size_t)bh * N + s0 + row) * kD + c8);
      *(uint4*)(sY + toff(row, c8)) = x;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const v8bf ah = tr_op<false>(sOh, 16 * k, 32 * w, l), al = tr_op<false>(sOl, 16 * k, 32 * w, l);
#pragma unroll
      for (int ft = 0; ft < 4; ++ft) {
        const v8bf by = tr_op<false>(sY, 16 * k, 32 * ft, l);
        acc[ft] = mfma(ah, by, acc[ft]);
        acc[ft] = mfma(al, by, acc[ft]);
      }
    }
  }
  // acc[ft][r] = partial[e = 32 w + acc_row(r)][f = 32 ft + l % 32]
  float* out = part + ((size_t)bh * n_chunks + ch) * kD * kD;
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(32 * w + acc_row(r)) * kD + 32 * ft + (l & 31)] = acc[ft][r];
}

__global__ __launch_bounds__(256) void kb_dw_sum1(const float* __restrict__ part, float* __restrict__ seg, int n_parts) {
  const int x = blockIdx.x * 256 + threadIdx.x, sg = blockIdx.y;
  const int per = (n_parts + kDwSeg - 1) / kDwSeg, p0 = sg * per, p1 = min(n_parts, p0 + per);
  float s = 0.f;
  for (int p = p0; p < p1; ++p) s += part[(size_t)p * kD * kD + x];
  seg[(size_t)sg * kD * kD + x] = s;
}

__global__ __launch_bounds__(256) void kb_dw_sum2(const float* __restrict__ seg, float* __restrict__ dw) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  float s = 0.f;
  for (int sg = 0; sg < kDwSeg; ++sg) s += seg[(size_t)sg * kD * kD + x];
  dw[x] = s;
}

// ---------------------------------------------------------------------------------------------------------
// Backward of the RMSNorm before the path (straight-through roundings). For Q (z = 0) and K (z = 1), with g the
// attention's gradient at the normalized values (fp32, in the dq / dk buffers), per token with its n = H*D
// channels and r = fp32(1 / sqrt(sum x^2 / n + eps)) as in the forward:
//   dx_c = r w_c g_c - x_c r^3 / n * s,  s = sum_c x_c w_c g_c;   dw_c = sum over tokens of x_c r g_c
// kb_norm_stats: grid (ceil(N / 8), B, 2), 512 threads, a wave per token: r and s (fp64 sums) -> rs[z][b][n][2].
// kb_norm_dw: grid (ceil(n / 256), n_chunks, 2 B): thread = channel, partial over a chunk of kNormChunk tokens in
// ascending order; kb_norm_dw_sum adds the partials in (b, chunk) order. kb_norm_dx then overwrites g with dx.
// ---------------------------------------------------------------------------------------------------------
constexpr int kNormChunk = 1024;

__global__ __launch_bounds__(512) void kb_norm_stats(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
                                                     const float* __restrict__ dq, const float* __restrict__ dk,
                                                     float* __restrict__ rs, int B, int H, int N, float eps) {
  const int z = blockIdx.z, b = blockIdx.y, l = threadIdx.x & 63;
  const int n = blockIdx.x * 8 + (threadIdx.x >> 6);
  if (n >= N) return;  // no barrier below
  const size_t row0 = ((size_t)b * H * N + n) * kD;
  const uint16_t* x = (z ? k : q) + row0;
  const float* g = (z ? dk : dq) + row0;
  const uint16_t* w = z ? wk : wq;
  double ss = 0.0, sg = 0.0;
  for (int h = 0; h < H; ++h) {
    const uint32_t xv = *(const uint32_t*)(x + (size_t)h * N * kD + 2 * l);
    const uint32_t wv = *(const uint32_t*)(w + h * kD + 2 * l);
    const float2 gv = *(const float2*)(g + (size_t)h * N * kD + 2 * l);
    const double x0 = bf16_lo(xv), x1 = bf16_hi(xv);
    ss += x0 * x0 + x1 * x1;
    sg += x0 * (double)bf16_lo(wv) * (double)gv.x + x1 * (double)bf16_hi(wv) * (double)gv.y;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    ss += __shfl_xor(ss, o);
    sg += __shfl_xor(sg, o);
  }
  if (l == 0) {
    const double m = ss / (double)(H * kD);
    float* o = rs + (((size_t)z * B + b) * N + n) * 2;
    o[0] = (float)(1.0 / sqrt(m + (double)eps));
    o[1] = (float)sg;
  }
}

__global__ __launch_bounds__(256) void kb_norm_dw(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                  const float* __restrict__ dq, const float* __restrict__ dk,
                                                  const float* __restrict__ rs, float* __restrict__ part, int B, int H,
                                                  int N, int n_chunks) {
  const int c = blockIdx.x * 256 + threadIdx.x, ch = blockIdx.y, z = blockIdx.z / B, b = blockIdx.z % B;
  if (c >= H * kD) return;
  const int h = c >> 7, d = c & 127;
  const int n0 = ch * kNormChunk, n1 = min(N, n0 + kNormChunk);
  const size_t hb = (((size_t)b * H + h) * N) * kD + d;
  const uint16_t* x = (z ? k : q) + hb;
  const float* g = (z ? dk : dq) + hb;
  const float* r = rs + (((size_t)z * B + b) * N) * 2;
  float acc = 0.f;
  for (int n = n0; n < n1; ++n) acc = fmaf(bf16_lo(x[(size_t)n * kD]) * r[2 * n], g[(size_t)n * kD], acc);
  part[(((size_t)z * B + b) * n_chunks + ch) * H * kD + c] = acc;
}

__global__ __launch_bounds__(256) void kb_norm_dw_sum(const float* __restrict__ part, float* __restrict__ dwq,
                                                      float* __restrict__ dwk, int B, int H, int n_chunks) {
  const int c = blockIdx.x * 256 + threadIdx.x, z = blockIdx.y;
  if (c >= H * kD) return;
  float acc = 0.f;
  for (int i = 0; i < B * n_chunks; ++i) acc += part[((size_t)z * B * n_chunks + i) * H * kD + c];
  (z ? dwk : dwq)[c] = acc;
}

__global__ __launch_bounds__(256) void kb_norm_dx(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
                                                  float* __restrict__ dq, float* __restrict__ dk,
                                                  const float* __restrict__ rs, int B, int H, int N) {
  const int z = blockIdx.y;
  const size_t e4 = (size_t)blockIdx.x * 256 + threadIdx.x;  // a group of 4 channels of one head row
  const size_t total4 = (size_t)B * H * N * (kD / 4);
  if (e4 >= total4) return;
  const int d4 = (int)(e4 % (kD / 4));
  const size_t rowi = e4 / (kD / 4);  // (b, h, n)
  const int n = (int)(rowi % N), h = (int)((rowi / N) % H), b = (int)(rowi / ((size_t)N * H));
  const uint2 xv = *(const uint2*)((z ? k : q) + rowi * kD + 4 * d4);
  const uint2 wv = *(const uint2*)((z ? wk : wq) + h * kD + 4 * d4);
  float* gp = (z ? dk : dq) + rowi * kD + 4 * d4;
  const float4 gv = *(const float4*)gp;
  const float* rr = rs + (((size_t)z * B + b) * N + n) * 2;
  const float r = rr[0], sc = r * r * r * rr[1] / (float)(H * kD);
  const float xs[4] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
  const float ws[4] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y)};
  const float gs[4] = {gv.x, gv.y, gv.z, gv.w};
  float o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = fmaf(r * ws[i], gs[i], -xs[i] * sc);
  *(float4*)gp = make_float4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------------------------------------
size_t kbq_lds_bytes() { return (size_t)4 * kTileBytes; }
size_t kbkv_lds_bytes() { return (size_t)4 * kTileBytes + 2 * 64 * 4; }
size_t kblinq_lds_bytes() { return (size_t)8 * kTileBytes + 3 * kD * 4; }
size_t kblink_lds_bytes() { return (size_t)6 * kTileBytes + kD * 4; }

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
  const int n_qbw = (p.n_qb + 31) / 32, n_kbw = (p.n_kb + 31) / 32;
  hipError_t e = launch_fill_f32((float*)b.sel_bits, (size_t)p.BH * p.n_kb * n_qbw, 0.f, s);
  if (e == hipSuccess) e = launch_fill_f32((float*)b.sel_bits_q, (size_t)p.BH * p.n_qb * n_kbw, 0.f, s);
  if (e != hipSuccess) return e;
  if (p.topk > 0) {
    hipLaunchKernelGGL(kb_sel, dim3(p.n_qb, p.BH), dim3(64), 0, s, p.block_idx, b.sel_bits, b.sel_bits_q, p.n_qb,
                       p.n_kb, p.topk, n_qbw, n_kbw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kb_q, dim3(p.n_qb, p.BH), dim3(256), kbq_lds_bytes(), s, b.q, b.k, b.v, b.dy, b.sel_bits_q,
                     b.lse, b.dd, b.dq, p.N, p.n_qb, n_kbw, p.blk_q, p.sm_scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kb_kv, dim3(p.n_kb, p.BH), dim3(256), kbkv_lds_bytes(), s, b.q, b.k, b.v, b.dy, b.sel_bits,
                     b.lse, b.dd, b.dk, b.dv, p.N, p.n_kb, n_qbw, p.blk_q, p.sm_scale);
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
  const int n_qbw = (p.n_qb + 31) / 32, kpad = mask_row_pad(p.n_kb);
  const size_t n_keep = (size_t)p.BH * n_qbw * kpad;
  hipLaunchKernelGGL(kb_keep_t, dim3((unsigned)((n_keep + 255) / 256)), dim3(256), 0, s, b.sel_bits, b.keep_t, p.n_qb,
                     p.n_kb, n_qbw, kpad, n_keep);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_state_sum(b.dhm, b.keep_t, b.dhj, p.n_kb, p.n_qb, kpad, p.BH, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(kb_lin_k, dim3(p.n_kb, p.BH), dim3(512), kblink_lds_bytes(), s, b.k, b.v, b.dhj, b.dk, b.dv,
                     p.N, p.n_kb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int n_chunks = (p.N + kDwChunk - 1) / kDwChunk;
  hipLaunchKernelGGL(kb_dw, dim3(n_chunks, p.BH), dim3(256), 0, s, b.o_l, b.dy, b.dw_part, p.N, n_chunks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kb_dw_sum1, dim3(kD * kD / 256, kDwSeg), dim3(256), 0, s, b.dw_part, b.dw_seg, p.BH * n_chunks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kb_dw_sum2, dim3(kD * kD / 256), dim3(256), 0, s, b.dw_seg, b.dw);
  return hipGetLastError();
}

size_t backward_dw_chunks(int N) { return (size_t)(N + kDwChunk - 1) / kDwChunk; }
size_t backward_norm_chunks(int N) { return (size_t)(N + kNormChunk - 1) / kNormChunk; }

hipError_t launch_norm_backward(const BwdPlan& b, const uint16_t* q_raw, const uint16_t* k_raw, float* dwq,
                                float* dwk, hipStream_t s) {
  const Plan& p = *b.fwd;
  const uint16_t* wq = (const uint16_t*)p.q_norm_w;
  const uint16_t* wk = (const uint16_t*)p.k_norm_w;
  hipLaunchKernelGGL(kb_norm_stats, dim3((p.N + 7) / 8, p.B, 2), dim3(512), 0, s, q_raw, k_raw, wq, wk, b.dq, b.dk,
                     b.norm_rs, p.B, p.H, p.N, p.norm_eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_chunks = (int)backward_norm_chunks(p.N), nch = p.H * kD;
  hipLaunchKernelGGL(kb_norm_dw, dim3((nch + 255) / 256, n_chunks, 2 * p.B), dim3(256), 0, s, q_raw, k_raw, b.dq,
                     b.dk, b.norm_rs, b.norm_part, p.B, p.H, p.N, n_chunks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kb_norm_dw_sum, dim3((nch + 255) / 256, 2), dim3(256), 0, s, b.norm_part, dwq, dwk, p.B, p.H,
                     n_chunks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t total4 = (size_t)p.B * p.H * p.N * (kD / 4);
  hipLaunchKernelGGL(kb_norm_dx, dim3((unsigned)((total4 + 255) / 256), 2), dim3(256), 0, s, q_raw, k_raw, wq, wk,
                     b.dq, b.dk, b.norm_rs, p.B, p.H, p.N);
  return hipGetLastError();
}
size_t backward_dw_segments() { return kDwSeg; }

}  // namespace sagesla
