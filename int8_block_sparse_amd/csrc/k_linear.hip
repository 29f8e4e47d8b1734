// K4: the linear branch of SLA over the non-selected key blocks (gfx950).
//
// "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn), §三(二) SLA item 2: the blocks that are not
// selected are modelled with linear-complexity attention followed by a linear projection. With phi = elu + 1
// on the raw bf16 q and k, per key block J the state is H_J = phi(K_J)^T V_J (D×D) and Z_J = sum phi(K_J) (D);
// the totals over all blocks are formed once and each query block subtracts its selected blocks' states:
//   O_l[i] = phi(q_i) H_m / (phi(q_i) . Z_m),  H_m = sum_J H_J - sum_{J selected} H_J,  out += O_l W_p.
// The projection is linear and the denominator is a scalar per row, so O_l W_p = (phi(q_i) H_m W_p) / den: the
// per-block states and their gather stay in the D×D state space and W_p is applied once per query block, to the
// product phi(Q_I) H_m, in the attention kernel's epilogue (k_attn.hip), which adds O_l W_p to the sparse part.
//
// Kernels:
//   k4_prep_wp   W_p^T with the MFMA key-slot order, bf16 (32 KB, once per call)
//   k4_states    per key block: H_J^T and Z_J into a column-tiled fp32 table (MFMA, HBM-bound; the backward).
//                The forward's fp16 table is written by the quantization kernel (k1_quant, k_quant.hip), whose
//                key-block workgroups already hold each block's V rows.
//   k4_mask      per query block: bitmask of the key blocks it did not select
//   k4_gemm      H_m = sum of the states of the unselected blocks, as the dense product keep-mask x table
//                (bf16 MFMA; about 90% of the mask is ones at 10% top-k); k4_gemm16 the same over the fp16 table
// (the attention kernel's epilogue then forms O_lin = (phi(Q) H_m) W_p / (phi(Q) . Z_m) per query block, MFMA)
// fp32 values enter the bf16 MFMAs as hi + lo bf16 pairs, so every product keeps ~16 significant bits.
#include "device_common.h"
#include "internal.h"
#include "lin_common.h"

namespace sagesla {

// W_p^T, positions permuted by slot_pos16: wpt[f][p], p = slot_pos16 applied within each 16 of e, in the swizzled
// plane layout (a straight copy into LDS)
__global__ __launch_bounds__(256) void k4_prep_wp(const uint16_t* __restrict__ wp, uint16_t* __restrict__ wpt) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // 16384 elements
  const int e = i >> 7, f = i & 127;             // wp[e][f]
  const int p = (e & ~15) | slot_pos16(e & 15);
  wpt[out_off(f, p) >> 1] = wp[i];
}

// ---------------------------------------------------------------------------------------------------------
// k4_states: grid (n_kb, BH), 256 threads (4 waves).
// LDS holds phi(K)^T (hi, lo) and V^T as [channel][key] bf16 rows of 128 B, 16-byte chunks XOR-swizzled.
// Wave w computes H^T[e][c] = sum_key v[e] phi(k)[c] for all e and c in [32w, 32w+32) (A = V^T, B = phi(K)).
// Table column x = e*128 + c; tile (x >> lxw) holds xw consecutive columns of every block: since xw <= 128 divides
// 128, the address of (e, c) is a per-lane part (c, J) plus e * 128 * n_kb floats. The forward uses xw = 128:
// each block's state is 129 pieces of 512 B, and 32 consecutive blocks of one tile are 16 KB contiguous.
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
// k4_mask: one wave per (bh, I) row. Bit J of word J/32 is 1 iff query block I did not select key block J
// (bits past n_kb are 0). Built in LDS with atomic ANDs, so an index that occurs twice clears its bit once, as
// a set would. Stored word-major per head, mask[bh][word][I] with rows padded to qpad, so that one word of a
// run of query blocks is contiguous.
// ---------------------------------------------------------------------------------------------------------
constexpr int kMaskMaxWords = 640;  // 20480 key blocks

__global__ __launch_bounds__(64) void k4_mask(const int32_t* __restrict__ idx, uint32_t* __restrict__ mask,
                                             int n_qb, int n_kb, int topk, int n_kbw, int qpad) {
  __shared__ uint32_t m[kMaskMaxWords];
  const int row = blockIdx.x, l = threadIdx.x, bh = row / n_qb, I = row % n_qb;
  for (int w = l; w < n_kbw; w += 64) {
    const int left = n_kb - 32 * w;
    m[w] = left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
  }
  __syncthreads();
  const int32_t* in = idx + (size_t)row * topk;
  for (int j = l; j < topk; j += 64) {
    const int J = min(max(in[j], 0), n_kb - 1);
    atomicAnd(&m[J >> 5], ~(1u << (J & 31)));
  }
  __syncthreads();
  for (int w = l; w < n_kbw; w += 64) mask[((size_t)bh * n_kbw + w) * qpad + I] = m[w];
}

// 8 keep bits -> 8 bf16 (0 or 1.0), element i = bit i
__device__ __forceinline__ uint4 expand_bits8(uint32_t b) {
  uint32_t r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t p = (b >> (2 * k)) & 3u;
    r[k] = ((p & 1u) | ((p & 2u) << 15)) * 0x3F80u;
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// ---------------------------------------------------------------------------------------------------------
// k4_gemm: C[I][x] = sum_J keep[I][J] H[J][x] over all key blocks J (keep = the k4_mask bits), for the state
// columns x of the table (H^T then Z). D = A B with A = keep (I x J, exact 0/1 in bf16) and B = the table
// (J x x) as hi + lo bf16, fp32 accumulation.
// grid (kStateX / 128 column groups, ceil(n_qb / 640) query-block chunks, BH), 512 threads (8 waves).
// Step = 32 key blocks (two MFMA k-steps of 16) = one mask word per query block. At the start of step s the
// workgroup issues buffer loads to LDS of the [32][128] fp32 table slice of step s+3 (16 KB contiguous) and of
// the chunk's 640 mask words of step s+2; during step s the waves run its MFMAs and rebuild slice s+1 into B
// fragments (hi, lo). Each wave forms its own A operands in registers: the byte of its row's mask word for
// (sub-step, lane half) becomes 8 bf16 through one read of a 256-entry byte table (at ~90% ones most lanes
// read entry 0xFF, which the LDS broadcasts). One wait plus one barrier per step orders everything; the wait leaves the previous
// step's loads in flight, so every load has two steps to land. Slices, words and B fragments each rotate
// through three buffers, each its own LDS object, so the compiler can tell the buffers being filled from those
// being read.
// Wave w owns query tiles 5 (w / 2) .. +4 and column tiles 2 (w % 2), +1: 10 output tiles of 32 x 32, each A
// operand feeding 4 MFMAs.
// ---------------------------------------------------------------------------------------------------------
constexpr int kGemmIT = 20;  // query-block tiles of 32 per workgroup
constexpr int kGemmThreads = 512;
constexpr int kGemmRows = kGemmIT * 32;  // query blocks per workgroup; mask rows are padded to a multiple

// wait until at most N of this wave's vector-memory operations are in flight (and every LDS operation is done),
// then a workgroup barrier
__device__ __forceinline__ void wait_vmem_all_lin() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int N> __device__ __forceinline__ void gemm_sync() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4));  // vmcnt(N) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kGemmThreads, 1) void k4_gemm(const float* __restrict__ table,
                                                          const uint32_t* __restrict__ mask,
                                                          float* __restrict__ state_m, int n_qb, int n_kb,
                                                          int n_kbw, int qpad) {
  // three-slot rings: table slices [row][128] fp32, B fragments [sub][tile][lane], mask words
  __shared__ __attribute__((aligned(1024))) float s_st0[32 * 128], s_st1[32 * 128], s_st2[32 * 128];
  __shared__ __attribute__((aligned(1024))) uint4 s_bh0[2 * 4 * 64], s_bh1[2 * 4 * 64], s_bh2[2 * 4 * 64];
  __shared__ __attribute__((aligned(1024))) uint4 s_bl0[2 * 4 * 64], s_bl1[2 * 4 * 64], s_bl2[2 * 4 * 64];
  __shared__ __attribute__((aligned(1024))) uint32_t s_w0[kGemmRows + 128], s_w1[kGemmRows + 128],
      s_w2[kGemmRows + 128];
  __shared__ __attribute__((aligned(1024))) uint4 s_lut[256];  // byte -> 8 bf16 of 0 / 1.0, element i = bit i
  constexpr int n_xt = kStateX / 128;
  const int xg = blockIdx.x, ic = blockIdx.y, bh = blockIdx.z;
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, g = l >> 5, lr = l & 31;
  const int I0 = ic * kGemmRows;
  const int n_it = min(kGemmIT, (n_qb - I0 + 31) >> 5);
  const int nss = n_kbw;  // steps of 32 key blocks
  const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(table + (size_t)bh * n_xt * n_kb * 128), (short)0, n_xt * n_kb * 128 * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(mask + (size_t)bh * n_kbw * qpad), (short)0, n_kbw * qpad * 4, 0x00020000);
  if (t < 256) {
    uint32_t d[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) d[k] = ((t >> (2 * k)) & 1 ? 0x3F80u : 0u) | ((t >> (2 * k + 1)) & 1 ? 0x3F800000u : 0u);
    s_lut[t] = make_uint4(d[0], d[1], d[2], d[3]);
  }

  // mask words of step ss for the chunk's rows: 3 loads of 1 KB (768 words; the last 128 are slack, and the
  // descriptor bounds return 0 past the end)
  // (the lane part of every load offset is the loop-invariant l * 16; the rest is uniform and goes in soffset)
  const uint32_t lane16 = (uint32_t)l * 16u;
  auto dma_w = [&](int ss, uint32_t* dst) {
    if (w < 3)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (__attribute__((address_space(3))) void*)(dst + 256 * w), 16, lane16,
                                               (uint32_t)((ss * qpad + I0 + 256 * w) * 4), 0, 0);
  };
  // table slice of step ss: rows 32 ss .. +31 of column group xg ([row][128] fp32, 16 KB contiguous); wave w loads
  // rows 4w .. 4w+3, two adjacent rows per 1 KB load. Rows past n_kb, whose mask bits are 0, read the next column
  // group's (finite) rows, or lie past the descriptor's range for the last group and read as zeros.
  auto dma_st = [&](int ss, float* dst) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t base = (uint32_t)((xg * n_kb + 32 * ss + 4 * w + 2 * h) * 512);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (__attribute__((address_space(3))) void*)(dst + (4 * w + 2 * h) * 128),
                                               16, lane16, base, 0, 0);
    }
  };
  // B fragments of one step from a staging slice, in 2 pieces (sub-steps). Thread t = (column tile xt = t>>7,
  // fragment lane fl = (t>>1)&63, half h = t&1) takes rows 16 sub + 8 (fl>>5) + 4 h .. +3 of column 32 xt +
  // (fl&31) and writes 8 bytes of the hi and of the lo fragment: consecutive threads write consecutive 8-byte
  // pieces. The reads (b_load) are issued two slots before the split and the writes (b_store).
  const int b_xt = t >> 7, b_fl = (t >> 1) & 63, b_h = t & 1;
  auto b_load = [&](int sub, const float* __restrict__ st, float (&v)[4]) {
    const float* c = st + (16 * sub + 8 * (b_fl >> 5) + 4 * b_h) * 128 + 32 * b_xt + (b_fl & 31);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = c[128 * k];
  };
  auto b_store = [&](int sub, const float (&v)[4], uint4* bh_, uint4* bl_) {
    uint32_t h01, l01, h23, l23;
    split2(v[0], v[1], h01, l01);
    split2(v[2], v[3], h23, l23);
    const int fi = (sub * 4 + b_xt) * 64 + b_fl;
    ((uint2*)&bh_[fi])[b_h] = make_uint2(h01, h23);
    ((uint2*)&bl_[fi])[b_h] = make_uint2(l01, l23);
  };
  auto build_b = [&](int sub, const float* __restrict__ st, uint4* bh_, uint4* bl_) {
    float v[4];
    b_load(sub, st, v);
    b_store(sub, v, bh_, bl_);
  };
  // A operand: byte (2 sub + g) of the row's word -> 8 bf16 from the byte table (mostly 0xFF: broadcast reads)
  auto a_frag = [&](uint32_t word, int sub) {
    const uint32_t b = (word >> (16 * sub + 8 * g)) & 0xFFu;
    return __builtin_bit_cast(v8bf, s_lut[b]);
  };

  // wave w: query tiles 5 (w / 2) .. +4, column tiles 2 (w % 2), +1; acc[2 q + c]
  const int wit = 5 * (w >> 1), wxt = 2 * (w & 1);
  v16f acc[10];
#pragma unroll
  for (int k = 0; k < 10; ++k) acc[k] = (v16f){};

  // one step with static buffers
  auto step = [&](int ss, const uint32_t* __restrict__ W, const uint4* __restrict__ Bh, const uint4* __restrict__ Bl,
                  const float* __restrict__ st_next, uint4* __restrict__ bh_next, uint4* __restrict__ bl_next,
                  uint32_t* __restrict__ w_fill, float* __restrict__ st_fill) {
    // Words ss and slice ss+1 (issued two steps back) have landed and B(ss) is built; the loads this wave
    // issued in step ss-1 (slice ss+2, words ss+1) may stay in flight. The buffers filled below are free. The
    // loads are issued even past the last step (they then read zeros or finite rows that no mask bit selects),
    // so that every wave has a fixed count in flight.
    if (ss == 0)
      gemm_sync<0>();
    else if (w < 3)
      gemm_sync<3>();
    else
      gemm_sync<2>();
    dma_st(ss + 3, st_fill);
    dma_w(ss + 2, w_fill);
    uint32_t wq[5];
#pragma unroll
    for (int q = 0; q < 5; ++q) wq[q] = W[32 * (wit + q) + lr];
    v8bf bhi[2][2], blo[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bhi[sub][c] = __builtin_bit_cast(v8bf, Bh[(sub * 4 + wxt + c) * 64 + l]);
        blo[sub][c] = __builtin_bit_cast(v8bf, Bl[(sub * 4 + wxt + c) * 64 + l]);
      }
    // 10 slots (sub, q): 4 MFMAs (2 column tiles x hi/lo) on the A operand formed two slots before
    v8bf af[10];
    float bv[4];  // staging values of the B build in flight
#pragma unroll
    for (int i = 0; i < 2; ++i) af[i] = a_frag(wq[i % 5], i / 5);
#pragma unroll
    for (int i = 0; i < 10; ++i) {  // tiles past n_it have zero words, never stored
      __builtin_amdgcn_sched_barrier(0);
      const int sub = i / 5, q = i % 5;
      if (i + 2 < 10) af[i + 2] = a_frag(wq[(i + 2) % 5], (i + 2) / 5);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        acc[2 * q + c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bhi[sub][c], acc[2 * q + c], 0, 0, 0);
        acc[2 * q + c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], blo[sub][c], acc[2 * q + c], 0, 0, 0);
      }
      // B fragments of step ss+1 (past the end: unused): reads in slots 0 and 5, split and writes in 2 and 7
      if (i == 0 || i == 5) b_load(i / 5, st_next, bv);
      if (i == 2 || i == 7) b_store(i / 5, bv, bh_next, bl_next);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: slices 0-2, words 0-1; B fragments of step 0. Step ss keeps words ss in s_w[ss % 3], slice ss in
  // s_st[ss % 3] and B(ss) in s_b*[ss % 3]: it builds B(ss+1) from slice ss+1, and refills the slice slot of
  // ss (slice ss+3) and the word slot of ss-1 (words ss+2).
  dma_st(0, s_st0);
  dma_st(1, s_st1);
  dma_st(2, s_st2);
  dma_w(0, s_w0);
  dma_w(1, s_w1);
  gemm_sync<0>();
  build_b(0, s_st0, s_bh0, s_bl0);
  build_b(1, s_st0, s_bh0, s_bl0);
  for (int ss = 0; ss < nss; ss += 3) {
    step(ss, s_w0, s_bh0, s_bl0, s_st1, s_bh1, s_bl1, s_w2, s_st0);
    if (ss + 1 < nss) step(ss + 1, s_w1, s_bh1, s_bl1, s_st2, s_bh2, s_bl2, s_w0, s_st1);
    if (ss + 2 < nss) step(ss + 2, s_w2, s_bh2, s_bl2, s_st0, s_bh0, s_bl0, s_w1, s_st2);
  }

  // Store. acc[2q + c][r] is C[I][x] with I = I0 + 32 (wit + q) + 8(r/4) + 4g + r%4, x = 128 xg + 32 (wxt + c) + lr.
  // Column group xg < 128 is row e = xg of H_m^T: written as the bf16 hi and lo plane rows (out_off layout) of
  // each query block's state record [hi plane 32 KB][lo plane 32 KB][Z fp32 512 B]; ten half-rounds of 64 query
  // blocks go through LDS so that every store is a contiguous 16 B piece of a plane row.
  // Column group 128 is Z, stored as fp32.
  unsigned char* const sm_bytes = (unsigned char*)state_m;
  constexpr size_t kRec = (size_t)kStateX * 4;  // bytes per query block
  if (xg == kD) {
#pragma unroll
    for (int q = 0; q < 5; ++q)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int I = I0 + 32 * (wit + q) + 8 * (r >> 2) + 4 * g + (r & 3);
          if (wit + q < n_it && I < n_qb)
            *(float*)(sm_bytes + ((size_t)bh * n_qb + I) * kRec + 65536 + 4 * (32 * (wxt + c) + lr)) = acc[2 * q + c][r];
        }
    return;
  }
  // staging per half-round: 64 rows (two wave pairs' query tiles) x 128 columns, columns 0-63 in s_st0 and
  // 64-127 in s_st1 (16 KB each)
#pragma unroll
  for (int q = 0; q < 5; ++q)
#pragma unroll
    for (int hr = 0; hr < 2; ++hr) {
      __syncthreads();  // the step buffers (first round) / the previous round's staging are free
      if ((w >> 2) == hr) {
        float* hw_ = (w & 1) ? s_st1 : s_st0;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            hw_[(32 * ((w >> 1) & 1) + 8 * (r >> 2) + 4 * g + (r & 3)) * 64 + 32 * c + lr] = acc[2 * q + c][r];
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j) {  // 64 rows x 16 chunks of 8 columns
        const int u = t + kGemmThreads * j, row = u >> 4, k8 = u & 15;
        const int it = 5 * (2 * hr + (row >> 5)) + q, I = I0 + 32 * it + (row & 31);
        const float* src = (k8 < 8 ? s_st0 : s_st1) + row * 64 + 8 * (k8 & 7);
        const float4 x0 = *(const float4*)src, x1 = *(const float4*)(src + 4);
        uint32_t hi[4], lo[4];
        split2(x0.x, x0.y, hi[0], lo[0]);
        split2(x0.z, x0.w, hi[1], lo[1]);
        split2(x1.x, x1.y, hi[2], lo[2]);
        split2(x1.z, x1.w, hi[3], lo[3]);
        if (it < n_it && I < n_qb) {
          unsigned char* rec = sm_bytes + ((size_t)bh * n_qb + I) * kRec + out_off(xg, 8 * k8);
          *(uint4*)rec = make_uint4(hi[0], hi[1], hi[2], hi[3]);
          *(uint4*)(rec + 32768) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
      }
    }
}

// ---------------------------------------------------------------------------------------------------------
// k4_gemm16 (the forward): the same keep-mask x table product over the fp16 table (block_state16, k_quant.hip).
// Each block J carries its own power of two 2^e_J, so the mask operand is keep[I][J] * 2^(e_J - E), E = max_J e_J
// over the head (exact in fp16 down to 2^-24; a block more than 24 binades below the head's largest is dropped), and
// the sums are the remaining state times 2^-E, H_m and Z_m alike (the linear branch's quotient does not see the
// common factor).
// grid (kStateX / 128 column groups, ceil(n_qb / 640) query-block chunks, BH), 512 threads (8 waves).
// Step = 32 key blocks (two k-steps of 16) = one mask word per query block. Table slices (32 rows of 256 B) and
// the chunk's mask words are loaded into registers four steps ahead and written to a three-slot LDS ring (16-byte
// chunks swizzled by tswz) one step ahead; one barrier per step. The table operand comes straight from the slice
// by transposing reads; the mask operand is two reads from the step's pattern tables (per group of four key blocks,
// the nibble's 0 / scale patterns, built once per step).
// The table is the first operand, so the accumulators hold C^T: every lane holds runs of four consecutive columns
// of one query block. Wave w owns query tiles 5 (w / 2) .. +4 and column tiles 2 (w % 2), +1.
// The store writes each query block's row e = x of H_m^T as an fp16 plane row with its own factor (the row's
// largest magnitude set below 2^15; the two waves of a row trade their halves' maxima through LDS) straight from
// the registers, and the Z group as fp32. Plane rows are stored row-major over the query blocks (one workgroup's
// rows are contiguous); the factors and Z go to each query block's aux record.
// ---------------------------------------------------------------------------------------------------------
constexpr int kAExpMin = -24;  // the smallest A scale 2^d, an fp16 subnormal

__global__ __launch_bounds__(kGemmThreads, 1) void k4_gemm16(const uint16_t* __restrict__ table,
                                                            const int32_t* __restrict__ bexp,
                                                            const uint32_t* __restrict__ mask,
                                                            unsigned char* __restrict__ plane,
                                                            unsigned char* __restrict__ aux, int n_qb, int n_kb,
                                                            int n_kbw, int qpad) {
  // three-slot LDS rings (table slices of 32 rows of 256 B, mask words of the chunk's rows); slot 0 of the slices
  // is also the store's exchange buffer
  __shared__ __attribute__((aligned(1024))) unsigned char s_st0[8192], s_st1[8192], s_st2[8192];
  __shared__ __attribute__((aligned(1024))) uint32_t s_w0[2 * kGemmThreads], s_w1[2 * kGemmThreads],
      s_w2[2 * kGemmThreads];
  // Per step, the mask operand's patterns with the scales applied: for each group of four key blocks (eight per step)
  // a table nibble -> 4 fp16 (element i = bit i ? scale of block 4 q + i : 0), 16 entries of 8 B (128 B: the lanes'
  // reads of different entries never share a bank). Group q = 4 sub + 2 g + h (k-step sub, lane half g, nibble h)
  // sits at 640 sub + 384 g + 128 h, so the two lane halves of an operand read different banks too. Three slots, as
  // the table slices.
  constexpr int kLgSlot = 1280;
  __shared__ __attribute__((aligned(1024))) unsigned char s_lg0[kLgSlot], s_lg1[kLgSlot], s_lg2[kLgSlot];
  __shared__ __attribute__((aligned(16))) uint16_t s_asc[kMaxKeyBlocks + 64];  // fp16 2^(e_J - E)
  __shared__ int s_red[kGemmThreads / 64];
  constexpr int n_xt = kStateX / 128;
  const int xg = blockIdx.x, ic = blockIdx.y, bh = blockIdx.z;
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, g = l >> 5, lr = l & 31;
  const int I0 = ic * kGemmRows;
  const int n_it = min(kGemmIT, (n_qb - I0 + 31) >> 5);
  const int nss = n_kbw;  // steps of 32 key blocks
  const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(table + (size_t)bh * n_xt * n_kb * 128), (short)0, n_xt * n_kb * 256, 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(mask + (size_t)bh * n_kbw * qpad), (short)0, n_kbw * qpad * 4, 0x00020000);
  // the head's largest block exponent, then the A scales of every key block (0 past n_kb)
  const int32_t* be = bexp + (size_t)bh * n_kb;
  int emax = INT_MIN;
  for (int J = t; J < n_kb; J += kGemmThreads) emax = max(emax, be[J]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) emax = max(emax, __shfl_xor(emax, o));
  if (l == 0) s_red[w] = emax;
  __syncthreads();
  int E = s_red[0];
#pragma unroll
  for (int k = 1; k < kGemmThreads / 64; ++k) E = max(E, s_red[k]);
  for (int J = t; J < 32 * nss; J += kGemmThreads) {
    uint32_t h = 0;
    if (J < n_kb) {
      const int d = be[J] - E;  // <= 0
      h = d >= -14 ? (uint32_t)(d + 15) << 10 : d >= kAExpMin ? 1u << (d + 24) : 0u;
    }
    s_asc[J] = (uint16_t)h;
  }

  // Staging through registers: the data of step s is loaded at step s - 4 (ordinary buffer loads, checked against
  // the descriptors' ranges: past them a load reads zeros) and written to its LDS slot at step s - 1, so every wait
  // is on a register and covers exactly the load it needs, with the loads of two later steps still in flight.
  // Thread t loads the slice's 16-byte chunk t (row t / 16, chunk t % 16) and stores it at chunk position
  // (t % 16) ^ tswz(row), and two mask words (rows 2t, 2t + 1 of the chunk; the 640 rows of the chunk and 384 that
  // are not used, so that every thread issues the same loads). Rows past n_kb (their A is 0) read the next column
  // group's rows (finite) or, past the head's table, zeros.
  const int srow = t >> 4;
  const uint32_t sgoff = (uint32_t)(xg * n_kb * 256 + srow * 256 + (t & 15) * 16);
  const uint32_t slds = (uint32_t)(srow * 256 + (((t & 15) ^ tswz(srow)) << 4));
  const uint32_t wgoff = (uint32_t)((I0 + 2 * t) * 4);
  struct Stage {
    v4i st;
    uint2 wd;
  };
  auto load = [&](int ss, Stage& r) {
    r.st = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rt, sgoff + (uint32_t)(ss * 32 * 256), 0, 0));
    r.wd = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rm, wgoff + (uint32_t)(ss * qpad * 4), 0, 0));
  };
  auto put = [&](const Stage& r, unsigned char* __restrict__ st, uint32_t* __restrict__ wd) {
    *(v4i*)(st + slds) = r.st;
    *(uint2*)(wd + 2 * t) = r.wd;
  };

  const int wit = 5 * (w >> 1), wxt = 2 * (w & 1);
  v16f acc[10];
#pragma unroll
  for (int k = 0; k < 10; ++k) acc[k] = (v16f){};

  // the pattern tables of step ss (threads 0-127, one entry each)
  auto build = [&](int ss, unsigned char* __restrict__ lg) {
    if (t < 128) {
      const int q = t >> 4, n = t & 15;
      const uint16_t* sc = &s_asc[32 * ss + 4 * q];
      const uint32_t lo = ((n & 1) ? (uint32_t)sc[0] : 0u) | ((n & 2) ? (uint32_t)sc[1] << 16 : 0u);
      const uint32_t hi = ((n & 4) ? (uint32_t)sc[2] : 0u) | ((n & 8) ? (uint32_t)sc[3] << 16 : 0u);
      *(uint2*)(lg + 640 * (q >> 2) + 384 * ((q >> 1) & 1) + 128 * (q & 1) + 8 * n) = make_uint2(lo, hi);
    }
  };
  // lane half g reads the groups 4 sub + 2 g + h at 640 sub + 384 g + 128 h
  const uint32_t lg_lane = 384u * g;
  const uint32_t bsh = 8u * g;  // the lane half's first mask bit in a k-step's 16
  auto mma = [&](int ss, const uint32_t* __restrict__ W, const unsigned char* __restrict__ st,
                 const unsigned char* __restrict__ lg) {
    uint32_t wq[5];
#pragma unroll
    for (int q = 0; q < 5; ++q) wq[q] = W[32 * (wit + q) + lr];
    v8h bop[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int c = 0; c < 2; ++c) bop[sub][c] = __builtin_bit_cast(v8h, tr_col_op(st, 16 * sub, 32 * (wxt + c), l));
#pragma unroll
    for (int i = 0; i < 10; ++i) {  // tiles past n_it have garbage words, never stored
      const int sub = i / 5, q = i % 5;
      const uint32_t n0 = __builtin_amdgcn_ubfe(wq[q], bsh + 16 * sub, 4);
      const uint32_t n1 = __builtin_amdgcn_ubfe(wq[q], bsh + 16 * sub + 4, 4);
      const unsigned char* lgs = lg + lg_lane + 640 * sub;
      const uint2 m0 = *(const uint2*)(lgs + 8 * n0), m1 = *(const uint2*)(lgs + 128 + 8 * n1);
      const v8h a = __builtin_bit_cast(v8h, make_uint4(m0.x, m0.y, m1.x, m1.y));
#pragma unroll
      for (int c = 0; c < 2; ++c)
        acc[2 * q + c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bop[sub][c], a, acc[2 * q + c], 0, 0, 0);
    }
  };

  // Step ss: barrier; stage step ss + 1 from its registers into slot (ss + 1) % 3; refill those registers with step
  // ss + 4; products of step ss from slot ss % 3. Register sets and slots both rotate over three steps, so the main
  // loop runs whole groups of three with no conditions (loads past the last step read zeros or finite rows that no
  // mask bit selects) and the last one or two steps follow.
  Stage r0, r1, r2;
  load(0, r0);
  load(1, r1);
  load(2, r2);
  put(r0, s_st0, s_w0);
  __syncthreads();  // every block's scale is in s_asc
  build(0, s_lg0);
  load(3, r0);
  auto step = [&](int ss, Stage& nx, const uint32_t* __restrict__ W, const unsigned char* __restrict__ st,
                  const unsigned char* __restrict__ lg, unsigned char* __restrict__ st_next,
                  uint32_t* __restrict__ w_next, unsigned char* __restrict__ lg_next) {
    __syncthreads();
    put(nx, st_next, w_next);
    build(ss + 1, lg_next);
    load(ss + 4, nx);
    mma(ss, W, st, lg);
  };
  int ss = 0;
  for (; ss + 3 <= nss; ss += 3) {
    step(ss, r1, s_w0, s_st0, s_lg0, s_st1, s_w1, s_lg1);
    step(ss + 1, r2, s_w1, s_st1, s_lg1, s_st2, s_w2, s_lg2);
    step(ss + 2, r0, s_w2, s_st2, s_lg2, s_st0, s_w0, s_lg0);
  }
  if (ss < nss) step(ss, r1, s_w0, s_st0, s_lg0, s_st1, s_w1, s_lg1);
  if (ss + 1 < nss) step(ss + 1, r2, s_w1, s_st1, s_lg1, s_st2, s_w2, s_lg2);
  wait_vmem_all_lin();  // the loads past the last step have landed in their registers: nothing is in flight
  __syncthreads();  // every wave is done reading the slots reused below

  // Store. The products ran with the table as the first operand, so acc[2q + c][r] is C[I][x] for query block
  // I = I0 + 32 (wit + q) + lr and column x = 128 xg + 32 (wxt + c) + 8 (r / 4) + 4 g + r % 4: every lane holds runs
  // of four consecutive columns of one query block, which it stores as they stand.
  if (xg == kD) {  // Z_m, fp32: 16 B per run
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int I = I0 + 32 * (wit + q) + lr;
      if (wit + q >= n_it || I >= n_qb) continue;
      unsigned char* r0 = aux + ((size_t)bh * n_qb + I) * kAuxBytes + kAuxZ;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(float4*)(r0 + 4 * (32 * (wxt + c) + 8 * r4 + 4 * g)) =
              make_float4(acc[2 * q + c][4 * r4], acc[2 * q + c][4 * r4 + 1], acc[2 * q + c][4 * r4 + 2],
                          acc[2 * q + c][4 * r4 + 3]);
    }
    return;
  }
  // row e = xg of H_m^T of each query block: its largest magnitude over the 128 columns (64 in this wave: two
  // column tiles, the lane pair g = 0, 1; the other 64 in wave w ^ 1, traded through LDS), then the fp16 plane row
  // in 8-byte runs and the row's factor
  float* const s_mx = (float*)s_st0;  // [8 waves][5 q][32 lanes]
  float mx[5];
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[2 * q + c][r]));
    mx[q] = fmaxf(m, swap_halves_f32(m));
    if (g == 0) s_mx[(w * 5 + q) * 32 + lr] = mx[q];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const float m = fmaxf(mx[q], s_mx[((w ^ 1) * 5 + q) * 32 + lr]);
    const int I = I0 + 32 * (wit + q) + lr;
    if (wit + q >= n_it || I >= n_qb) continue;
    int kx = 0;
    (void)frexpf(m, &kx);  // m < 2^kx
    const int sh = 15 - kx;
    // the row's 256 B as the epilogue's LDS holds row xg of the plane (out_off with the row offset taken out)
    unsigned char* r0 = plane + (((size_t)bh * kD + xg) * n_qb + I) * 256 - (size_t)xg * 256;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const v4f x = {acc[2 * q + c][4 * r4], acc[2 * q + c][4 * r4 + 1], acc[2 * q + c][4 * r4 + 2],
                       acc[2 * q + c][4 * r4 + 3]};
        *(uint2*)(r0 + out_off(xg, 32 * (wxt + c) + 8 * r4 + 4 * g)) =
            make_uint2(pack_f16x2(ldexpf(x[0], sh), ldexpf(x[1], sh)), pack_f16x2(ldexpf(x[2], sh), ldexpf(x[3], sh)));
      }
    if (g == 0 && (w & 1) == 0)
      *(float*)(aux + ((size_t)bh * n_qb + I) * kAuxBytes + kAuxF + 4 * xg) = m > 0.f ? ldexpf(1.f, kx - 15) : 0.f;
  }
}

int mask_row_pad(int n_qb) { return (n_qb + kGemmRows - 1) / kGemmRows * kGemmRows; }

hipError_t launch_linear(const Plan& p, const uint16_t* k, const uint16_t* v, hipStream_t s) {
  hipLaunchKernelGGL(k4_prep_wp, dim3(kD * kD / 256), dim3(256), 0, s, (const uint16_t*)p.w_proj, p.wpt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.lin_precise) {  // the forward's fp16 table was written by the quantization kernel
    hipLaunchKernelGGL(k4_states, dim3(p.n_kb, p.BH), dim3(256), 0, s, k, v, p.state, p.N, p.n_kb, 7, kStateX / 128);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int rows = p.BH * p.n_qb, n_kbw = (p.n_kb + 31) / 32, qpad = mask_row_pad(p.n_qb);
  hipLaunchKernelGGL(k4_mask, dim3(rows), dim3(64), 0, s, p.block_idx, p.keep_mask, p.n_qb, p.n_kb, p.topk, n_kbw,
                     qpad);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.lin_precise) return launch_state_sum(p.state, p.keep_mask, p.state_m, p.n_qb, p.n_kb, qpad, p.BH, s);
  hipLaunchKernelGGL(k4_gemm16, dim3(kStateX / 128, qpad / kGemmRows, p.BH), dim3(kGemmThreads), 0, s, p.state16,
                     p.state_exp, p.keep_mask, p.plane16, p.aux16, p.n_qb, p.n_kb, n_kbw, qpad);
  return hipGetLastError();
}

hipError_t launch_state_sum(const float* table, const uint32_t* mask, float* out, int n_out, int n_in, int pad, int BH,
                            hipStream_t s) {
  hipLaunchKernelGGL(k4_gemm, dim3(kStateX / 128, pad / kGemmRows, BH), dim3(kGemmThreads), 0, s, table, mask, out,
                     n_out, n_in, (n_in + 31) / 32, pad);
  return hipGetLastError();
}

}  // namespace sagesla
