// K4: the linear branch of SLA over the non-selected key blocks (gfx950).
//
// "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn), §三(二) SLA item 2: the blocks that are not
// selected are modelled with linear-complexity attention followed by a linear projection. With phi = elu + 1
// on the raw bf16 q and k, per key block J the state is H_J = phi(K_J)^T V_J (D×D) and Z_J = sum phi(K_J) (D);
// the totals over all blocks are formed once and each query block subtracts its selected blocks' states:
//   O_l[i] = phi(q_i) H_m / (phi(q_i) . Z_m),  H_m = sum_J H_J - sum_{J selected} H_J,  out += O_l W_p.
// The projection is linear and the denominator is a scalar per row, so O_l W_p = (phi(q_i) H_m W_p) / den: the
// per-block states and their gather stay in the D×D state space and W_p is applied once per query block, to the
// product phi(Q_I) H_m, in the output kernel.
//
// Kernels:
//   k4_prep_wp   W_p^T with the MFMA key-slot order, bf16 (32 KB, once per call)
//   k4_states    per key block: H_J^T and Z_J into a column-tiled table (MFMA, HBM-bound)
//   k4_gather    per (b,h) and column tile: the tile of all blocks' states sits in LDS; totals once, then for
//                every query block H_m = total - sum over its selected blocks (LDS-bound)
//   k4_out       per query block: O_lin = (phi(Q) H_m) W_p / (phi(Q) . Z_m) (MFMA)
// fp32 values enter the bf16 MFMAs as hi + lo bf16 pairs, so every product keeps ~16 significant bits.
#include "device_common.h"
#include "internal.h"

namespace sagesla {

// position of key/channel slot inside a 16-group such that the MFMA 32x32x16 lane (half g, slot i) reads
// 8 consecutive positions: slot (g, i) <-> index 8*(i/4) + 4*g + (i%4); position 8*g + 4*(i/4) + (i%4).
__device__ __forceinline__ int slot_pos16(int off) {  // off = index within the 16-group
  return (off & 3) | ((off & 4) << 1) | ((off & 8) >> 1);
}

// W_p^T, positions permuted as above: wpt[f][p], p = slot_pos16 applied within each 16 of e.
__global__ __launch_bounds__(256) void k4_prep_wp(const uint16_t* __restrict__ wp, uint16_t* __restrict__ wpt) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // 16384 elements
  const int e = i >> 7, f = i & 127;             // wp[e][f]
  const int p = (e & ~15) | slot_pos16(e & 15);
  wpt[f * kD + p] = wp[i];
}

// phi(x) = elu(x) + 1: x + 1 for x > 0, e^x otherwise (hardware exp2 of x log2(e); the values then enter the
// MFMAs as hi + lo bf16 pairs, ~16 significant bits)
__device__ __forceinline__ float phi_f(float x) {
  return x > 0.f ? x + 1.f : __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// two fp32 values -> bf16 pairs hi = bf16(x) and lo = bf16(x - hi), packed as (x0, x1)
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(x0, x1);
  lo = pack_bf16x2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
}

constexpr int kRunUnroll = 8;              // runs per gather step
constexpr int kRunPad = 2 * kRunUnroll;    // zero runs after each row's last run: covers the next-step prefetch

__global__ void k_fill_i32(int32_t* __restrict__ d, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) d[i] = v;
}

// ---------------------------------------------------------------------------------------------------------
// k4_states: grid (n_kb, BH), 256 threads (4 waves).
// LDS holds phi(K)^T (hi, lo) and V^T as [channel][key] bf16 rows of 128 B, 16-byte chunks XOR-swizzled.
// Wave w computes H^T[e][c] = sum_key v[e] phi(k)[c] for all e and c in [32w, 32w+32) (A = V^T, B = phi(K)).
// Table column x = e*128 + c; tile (x >> lxw) holds xw consecutive columns of every block: since xw <= 128 divides
// 128, the address of (e, c) is a per-lane part (c, J) plus e * 128 * n_kb floats.
// ---------------------------------------------------------------------------------------------------------
__device__ __forceinline__ int lds_off(int row, int key) {  // byte offset of (row, key) in a [128][64] bf16 tile
  return row * 128 + (((key >> 3) ^ swz8(row)) << 4) + ((key & 7) << 1);
}

__global__ __launch_bounds__(256) void k4_states(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                float* __restrict__ table, int N, int n_kb, int lxw, int n_xt) {
  const int xw = 1 << lxw;
  __shared__ __attribute__((aligned(16))) unsigned char s_pkh[kD * 128];
  __shared__ __attribute__((aligned(16))) unsigned char s_pkl[kD * 128];
  __shared__ __attribute__((aligned(16))) unsigned char s_vt[kD * 128];
  __shared__ float s_z[16][kD + 1];
  const int J = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 5, lr = l & 31;
  const int cg = t & 15, kg = t >> 4;  // loader: channels 8cg..+7, keys 4kg..+3
  const size_t base = ((size_t)bh * N + (size_t)J * kBlkK) * kD;
  const int nv = min(kBlkK, N - J * kBlkK);

  // ---- load, phi, split, transpose into LDS
  uint32_t kw[4][4], vw[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int r = 4 * kg + b;
    uint4 a = make_uint4(0, 0, 0, 0), c = make_uint4(0, 0, 0, 0);
    if (r < nv) {
      a = *(const uint4*)(k + base + (size_t)r * kD + cg * 8);
      c = *(const uint4*)(v + base + (size_t)r * kD + cg * 8);
    }
    kw[b][0] = a.x; kw[b][1] = a.y; kw[b][2] = a.z; kw[b][3] = a.w;
    vw[b][0] = c.x; vw[b][1] = c.y; vw[b][2] = c.z; vw[b][3] = c.w;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = cg * 8 + e;
    float pk[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float x = (e & 1) ? bf16_hi(kw[b][e >> 1]) : bf16_lo(kw[b][e >> 1]);
      pk[b] = (4 * kg + b < nv) ? phi_f(x) : 0.f;
    }
    uint32_t h01, l01, h23, l23;
    split2(pk[0], pk[1], h01, l01);
    split2(pk[2], pk[3], h23, l23);
    const int off = lds_off(row, 4 * kg);
    *(uint2*)(s_pkh + off) = make_uint2(h01, h23);
    *(uint2*)(s_pkl + off) = make_uint2(l01, l23);
    // V^T: channel e of keys 4kg..4kg+3, bf16 bits moved as they are
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    *(uint2*)(s_vt + off) = make_uint2(__builtin_amdgcn_perm(vw[1][e >> 1], vw[0][e >> 1], sel),
                                       __builtin_amdgcn_perm(vw[3][e >> 1], vw[2][e >> 1], sel));
    s_z[kg][row] = (pk[0] + pk[1]) + (pk[2] + pk[3]);
  }
  __syncthreads();

  // ---- H^T = V^T phi(K): m = e (4 tiles), n = c (tile w), k = key (4 steps of 16)
  v16f acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = (v16f){};
  const int crow = 32 * w + lr;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int key = 16 * s + 8 * g;
    const v8bf bh_ = *(const v8bf*)(s_pkh + lds_off(crow, key));
    const v8bf bl_ = *(const v8bf*)(s_pkl + lds_off(crow, key));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const v8bf a = *(const v8bf*)(s_vt + lds_off(32 * mt + lr, key));
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh_, acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl_, acc[mt], 0, 0, 0);
    }
  }

  // ---- store H^T[e][c]: lane part (c, J, half g), row part e * 128 * n_kb floats
  const int c = crow;
  const size_t estride = (size_t)kD * n_kb;  // floats between rows e and e+1 of the table
  float* tl = table + (size_t)bh * n_xt * n_kb * xw + ((size_t)(c >> lxw) * n_kb + J) * xw + (c & (xw - 1)) +
              (size_t)(4 * g) * estride;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) tl[(size_t)(32 * mt + 8 * (r >> 2) + (r & 3)) * estride] = acc[mt][r];
  if (t < kD) {
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) z += s_z[j][t];
    const int x = kD * kD + t;
    table[(size_t)bh * n_xt * n_kb * xw + ((size_t)(x >> lxw) * n_kb + J) * xw + (x & (xw - 1))] = z;
  }
}

// ---------------------------------------------------------------------------------------------------------
// k4_runs: the selected blocks of each query block as runs of consecutive indices [a, b). One wave per
// (bh, I) row. For any list (sorted or not) the sum over its elements equals the sum over these runs of
// P[b] - P[a] with P the exclusive prefix sum over blocks; for the ascending selections of structured video
// inputs there are about a third as many runs as blocks. Runs are stored as LDS byte offsets of rows a and b
// in the gather kernel's prefix table (row stride xw floats).
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k4_runs(const int32_t* __restrict__ idx, int2* __restrict__ runs,
                                             int32_t* __restrict__ run_cnt, int n_kb, int topk, int rstride,
                                             int rows, int row_bytes) {
  const int row = blockIdx.x;
  if (row >= rows) return;
  const int l = threadIdx.x;
  const int32_t* in = idx + (size_t)row * topk;
  int2* out = runs + (size_t)row * rstride;
  int ns = 0, ne = 0;
  for (int j0 = 0; j0 < topk; j0 += 64) {
    const int j = j0 + l;
    const bool ok = j < topk;
    const int cur = ok ? min(max(in[j], 0), n_kb - 1) : 0;
    const int prev = (ok && j > 0) ? min(max(in[j - 1], 0), n_kb - 1) : -2;
    const int next = (ok && j + 1 < topk) ? min(max(in[j + 1], 0), n_kb - 1) : -2;
    const bool st = ok && cur != prev + 1;
    const bool en = ok && next != cur + 1;
    const unsigned long long ms = __ballot(st), me = __ballot(en);
    const unsigned long long lt = l ? (~0ull >> (64 - l)) : 0ull;
    if (st) out[ns + __popcll(ms & lt)].x = cur * row_bytes;
    if (en) out[ne + __popcll(me & lt)].y = (cur + 1) * row_bytes;
    ns += __popcll(ms);
    ne += __popcll(me);
  }
  // zero runs after the last one: the gather reads up to kRunPad - 1 entries past the count
  if (l < kRunPad) out[ns + l] = make_int2(0, 0);
  if (l == 0) run_cnt[row] = ns;
}

// ---------------------------------------------------------------------------------------------------------
// k4_gather: grid (n_xt, BH), 1024 threads (16 waves). LDS: the prefix table (n_kb + 1) * xw floats and 1024
// scan partials. xw is a power of two from 4 to 64 and divides the state size 16512.
// The state tile of all key blocks (xw columns) is loaded into LDS and turned in place into its exclusive
// prefix sum over blocks, P[0..n_kb] (P[n_kb] = the total over all blocks); the scan segments and their
// combination have a fixed order, so the result is deterministic. Each wave then serves ipw = 64/xw query
// blocks at once, each lane covering 4 consecutive columns:
//   H_m[x] = P[n_kb][x] - sum over the runs [a, b) of the query block's selection of (P[b][x] - P[a][x]).
// Run offsets are read 8 at a time into registers (one broadcast address per query block) with the next 8
// prefetched; run rows end in 8 zero runs, so these loads need no bounds test.
// ---------------------------------------------------------------------------------------------------------
constexpr int kGatherThreads = 1024;

__global__ __launch_bounds__(kGatherThreads) void k4_gather(const float* __restrict__ table,
                                                           const int2* __restrict__ runs,
                                                           const int32_t* __restrict__ run_cnt,
                                                           float* __restrict__ state_m, int n_qb, int n_kb,
                                                           int rstride, int xw, int n_xt) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float* P = lds;                              // [(n_kb + 1) * xw]
  float* seg = lds + (size_t)(n_kb + 1) * xw;  // [kGatherThreads]
  const int xt = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x;
  const float* src = table + ((size_t)bh * n_xt + xt) * n_kb * xw;
  const int nflt = n_kb * xw;
  for (int i = 4 * t; i < nflt; i += 4 * kGatherThreads) *(float4*)(P + i) = *(const float4*)(src + i);
  __syncthreads();
  {  // exclusive prefix over blocks: thread (sg, xi) scans rows [j0, j1) of column xi
    const int nseg = kGatherThreads / xw, sg = t / xw, xi = t % xw;
    const int per = (n_kb + nseg - 1) / nseg;
    const int j0 = min(n_kb, sg * per), j1 = min(n_kb, j0 + per);
    float run = 0.f;
    for (int j = j0; j < j1; ++j) run += P[j * xw + xi];
    seg[t] = run;
    __syncthreads();
    float off = 0.f;
    for (int s2 = 0; s2 < sg; ++s2) off += seg[s2 * xw + xi];
    for (int j = j0; j < j1; ++j) {
      const float v = P[j * xw + xi];
      P[j * xw + xi] = off;
      off += v;
    }
    if (sg == nseg - 1) P[n_kb * xw + xi] = off;  // empty trailing segments pass their offset on
    __syncthreads();
  }

  // gather: lane = (query block sub, 4 consecutive columns col4), one 16-byte LDS read per run endpoint
  const int w = t >> 6, l = t & 63;
  const int lpr = xw >> 2;  // lanes per query block
  const int ipw = 64 / lpr, sub = l / lpr, col4 = (l % lpr) * 4;
  const unsigned char* Pb = (const unsigned char*)P + col4 * 4;
  const float4 total = *(const float4*)(P + n_kb * xw + col4);
  const int x = xt * xw + col4;
  for (int I0 = w * ipw; I0 < n_qb; I0 += (kGatherThreads / 64) * ipw) {
    const int I = I0 + sub;
    if (I < n_qb) {
      const size_t row = (size_t)bh * n_qb + I;
      const int cnt = run_cnt[row];
      const int4* rr = (const int4*)(runs + row * rstride);  // two runs per int4; rows padded with zero runs
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      int4 cur[kRunUnroll / 2], nxt[kRunUnroll / 2];
#pragma unroll
      for (int i = 0; i < kRunUnroll / 2; ++i) cur[i] = rr[i];
      for (int r = 0; r < cnt; r += kRunUnroll) {  // r <= cnt - 1: the prefetch stays below cnt + kRunPad
#pragma unroll
        for (int i = 0; i < kRunUnroll / 2; ++i) nxt[i] = rr[(r + kRunUnroll) / 2 + i];
#pragma unroll
        for (int i = 0; i < kRunUnroll / 2; ++i) {  // zero runs add P[0] - P[0] = 0
          const float4 b0 = *(const float4*)(Pb + cur[i].y), a0 = *(const float4*)(Pb + cur[i].x);
          const float4 b1 = *(const float4*)(Pb + cur[i].w), a1 = *(const float4*)(Pb + cur[i].z);
          acc.x += (b0.x - a0.x) + (b1.x - a1.x);
          acc.y += (b0.y - a0.y) + (b1.y - a1.y);
          acc.z += (b0.z - a0.z) + (b1.z - a1.z);
          acc.w += (b0.w - a0.w) + (b1.w - a1.w);
        }
#pragma unroll
        for (int i = 0; i < kRunUnroll / 2; ++i) cur[i] = nxt[i];
      }
      *(float4*)(state_m + row * kStateX + x) =
          make_float4(total.x - acc.x, total.y - acc.y, total.z - acc.z, total.w - acc.w);
    }
  }
}

// ---------------------------------------------------------------------------------------------------------
// k4_out: one workgroup (4 waves) per (bh, I) query block.
//   U^T[e][i] = sum_c H_m^T[e][c] phi(Q)^T[c][i]        (A = H_m^T hi/lo from LDS, B = phi(Q) hi/lo in registers)
//   O^T[f][i] = sum_e W_p^T[f][e] U^T[e][i] / den[i]     (A = W_p^T from LDS, B = U^T hi/lo from the accumulators)
// with den[i] = phi(q_i) . Z_m. The block's remaining state is loaded once into LDS as bf16 hi and lo planes
// ([e][c] rows of 256 B, 16-byte chunks XOR-swizzled by e); after the first product the hi plane's space takes
// W_p^T. Wave w handles its own 32 rows. Products hi*hi + hi*lo + lo*hi keep ~16 significant bits.
// ---------------------------------------------------------------------------------------------------------
__device__ __forceinline__ int out_off(int e, int c) {  // byte offset of (e, c) in one [128][128] bf16 plane
  return e * 256 + ((((c >> 3) ^ e) & 15) << 4) + ((c & 7) << 1);
}

template <int BLKQ>
__global__ __launch_bounds__(BLKQ * 2) void k4_out(const uint16_t* __restrict__ q, const float* __restrict__ state_m,
                                                  const uint16_t* __restrict__ wpt, float* __restrict__ o_lin, int N,
                                                  int n_qb, int total) {
  constexpr int NT = BLKQ * 2;
  __shared__ __attribute__((aligned(16))) unsigned char s_hi[kD * 256];
  __shared__ __attribute__((aligned(16))) unsigned char s_lo[kD * 256];
  __shared__ float s_z[kD];
  const int item = xcd_remap(blockIdx.x, total);
  const int bh = item / n_qb, I = item % n_qb;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 5, lr = l & 31;
  const float* sm = state_m + ((size_t)bh * n_qb + I) * kStateX;

  // stage: 8 consecutive floats of one row e per thread per step
  for (int u = t; u < kD * kD / 8; u += NT) {
    const int e = u >> 4, c0 = (u & 15) * 8;
    const float4 a0 = *(const float4*)(sm + e * kD + c0);
    const float4 a1 = *(const float4*)(sm + e * kD + c0 + 4);
    uint32_t hw[4], lw[4];
    split2(a0.x, a0.y, hw[0], lw[0]);
    split2(a0.z, a0.w, hw[1], lw[1]);
    split2(a1.x, a1.y, hw[2], lw[2]);
    split2(a1.z, a1.w, hw[3], lw[3]);
    *(uint4*)(s_hi + out_off(e, c0)) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *(uint4*)(s_lo + out_off(e, c0)) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  if (t < kD) s_z[t] = sm[kD * kD + t];
  __syncthreads();

  const int row = I * BLKQ + 32 * w + lr;
  const bool rok = row < N;
  const uint16_t* qrow = q + ((size_t)bh * N + (rok ? row : 0)) * kD;
  v8bf bqh[8], bql[8];
  float den = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c0 = 16 * s + 8 * g;
    uint4 wq = make_uint4(0, 0, 0, 0);
    if (rok) wq = *(const uint4*)(qrow + c0);
    const uint32_t ww[4] = {wq.x, wq.y, wq.z, wq.w};
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float p0 = phi_f(bf16_lo(ww[u])), p1 = phi_f(bf16_hi(ww[u]));
      den = fmaf(p0, s_z[c0 + 2 * u], den);
      den = fmaf(p1, s_z[c0 + 2 * u + 1], den);
      split2(p0, p1, hw[u], lw[u]);
    }
    bqh[s] = __builtin_bit_cast(v8bf, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    bql[s] = __builtin_bit_cast(v8bf, make_uint4(lw[0], lw[1], lw[2], lw[3]));
  }
  den += swap_halves_f32(den);
  const float inv = 1.f / den;

  // ---- U^T = H_m^T phi(Q)^T
  v16f acc[4];
#pragma unroll
  for (int et = 0; et < 4; ++et) {
    acc[et] = (v16f){};
    const int e = 32 * et + lr;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int off = out_off(e, 16 * s + 8 * g);
      const v8bf ah = *(const v8bf*)(s_hi + off);
      const v8bf al = *(const v8bf*)(s_lo + off);
      acc[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bqh[s], acc[et], 0, 0, 0);
      acc[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bql[s], acc[et], 0, 0, 0);
      acc[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bqh[s], acc[et], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with the state planes
  // W_p^T (bf16, rows f of 256 B, already in MFMA slot order along e) into the hi plane's space, same swizzle
  for (int u = t; u < kD * kD / 8; u += NT) {
    const int f = u >> 4, e0 = (u & 15) * 8;
    *(uint4*)(s_hi + out_off(f, e0)) = *(const uint4*)(wpt + f * kD + e0);
  }
  __syncthreads();

  // ---- O^T = W_p^T U^T: B operand slot (g, i) of step s2 is e = 16 s2 + 8(i/4) + 4g + i%4, i.e. accumulator
  // register 8(s2%2) + i of tile s2/2 in this lane; W_p^T rows hold e in the matching permuted order.
  v16f acc2[4];
#pragma unroll
  for (int ft = 0; ft < 4; ++ft) acc2[ft] = (v16f){};
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) {
    const int src = s2 >> 1, r0 = 8 * (s2 & 1);
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) split2(acc[src][r0 + 2 * u], acc[src][r0 + 2 * u + 1], hw[u], lw[u]);
    const v8bf bhi = __builtin_bit_cast(v8bf, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    const v8bf blo = __builtin_bit_cast(v8bf, make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
    for (int ft = 0; ft < 4; ++ft) {
      const v8bf a = *(const v8bf*)(s_hi + out_off(32 * ft + lr, 16 * s2 + 8 * g));
      acc2[ft] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bhi, acc2[ft], 0, 0, 0);
      acc2[ft] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, blo, acc2[ft], 0, 0, 0);
    }
  }
  if (rok) {
    float* orow = o_lin + ((size_t)bh * N + row) * kD;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f0 = 32 * ft + 8 * r4 + 4 * g;
        *(float4*)(orow + f0) = make_float4(acc2[ft][4 * r4] * inv, acc2[ft][4 * r4 + 1] * inv,
                                            acc2[ft][4 * r4 + 2] * inv, acc2[ft][4 * r4 + 3] * inv);
      }
  }
}

int run_stride(int topk) { return ((topk + 1) & ~1) + kRunPad; }

size_t gather_lds_bytes(int n_kb, int xw) { return ((size_t)(n_kb + 1) * xw + kGatherThreads) * sizeof(float); }

hipError_t launch_linear(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v, hipStream_t s) {
  hipLaunchKernelGGL(k4_prep_wp, dim3(kD * kD / 256), dim3(256), 0, s, (const uint16_t*)p.w_proj, p.wpt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int lxw = __builtin_ctz(p.state_xw);
  hipLaunchKernelGGL(k4_states, dim3(p.n_kb, p.BH), dim3(256), 0, s, k, v, p.state, p.N, p.n_kb, lxw,
                     p.n_state_xt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t lds = gather_lds_bytes(p.n_kb, p.state_xw);
  static bool attr_set = false;  // raising the dynamic-LDS cap is idempotent; racing first calls are harmless
  if (!attr_set) {
    e = hipFuncSetAttribute((const void*)k4_gather, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int rows = p.BH * p.n_qb;
  if (p.topk > 0) {
    hipLaunchKernelGGL(k4_runs, dim3(rows), dim3(64), 0, s, p.block_idx, p.runs, p.run_cnt, p.n_kb, p.topk,
                       run_stride(p.topk), rows, p.state_xw * (int)sizeof(float));
  } else {  // nothing selected: every row has zero runs (and its padding must still read as zero runs)
    hipLaunchKernelGGL(k_fill_i32, dim3((rows + 255) / 256), dim3(256), 0, s, p.run_cnt, rows, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_fill_i32, dim3((rows * 2 * run_stride(0) + 255) / 256), dim3(256), 0, s, (int32_t*)p.runs,
                       rows * 2 * run_stride(0), 0);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k4_gather, dim3(p.n_state_xt, p.BH), dim3(kGatherThreads), lds, s, p.state, p.runs, p.run_cnt,
                     p.state_m, p.n_qb, p.n_kb, run_stride(p.topk), p.state_xw, p.n_state_xt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int total = p.BH * p.n_qb;
  if (p.blk_q == 128)
    hipLaunchKernelGGL(k4_out<128>, dim3(total), dim3(256), 0, s, q, p.state_m, p.wpt, p.o_lin, p.N, p.n_qb,
                       total);
  else
    hipLaunchKernelGGL(k4_out<64>, dim3(total), dim3(128), 0, s, q, p.state_m, p.wpt, p.o_lin, p.N, p.n_qb,
                       total);
  return hipGetLastError();
}

}  // namespace sagesla
