// W8A8 block-quantized linear layer (gfx950): Y = X W^T + b with 8-bit codes and one fp32 scale per 128×128
// block of each matrix.
//
// "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn), §三(四) item 1: weights in independent 128×128
// blocks with their own quantization parameters, activations quantized dynamically with clipping; the
// TurboDiffusion release news (chooseai.net) quantizes parameters and activations alike in 128×128 blocks.
//
//   k5_quant  one 128×128 block per workgroup: absmax, t = fp32(clip * absmax), s = fp32(t / 127), codes
//   k5_gemm   Y^T tiles on v_mfma_i32_32x32x32_i8: per k-block (128 input features) the exact int32 partial
//             P_kb, then y = fma(P_kb, fp32(s_x * s_w), y) in fp32, ascending k-blocks; bf16 output
#include "device_common.h"
#include "internal.h"

namespace sagesla {

typedef __attribute__((address_space(3))) void w_lds_void;

// ---------------------------------------------------------------------------------------------------------
// k5_quant: grid (cols / 128, ceil(rows / 128)), 256 threads. Thread t owns columns 8 (t % 16) .. +7 of rows
// t / 16 + 16 i (i < 8): a wave covers 4 whole 256-byte row pieces per load.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k5_quant(const uint16_t* __restrict__ x, int rows, int cols, float clip,
                                                int8_t* __restrict__ codes, float* __restrict__ scales) {
  const int kb = blockIdx.x, mb = blockIdx.y;
  const int t = threadIdx.x, cg = t & 15, rl = t >> 4;
  const int r0 = mb * 128, nr = min(128, rows - r0);
  const uint16_t* src = x + (size_t)r0 * cols + kb * 128 + cg * 8;
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rl + 16 * i;
    raw[i] = (r < nr) ? *(const uint4*)(src + (size_t)r * cols) : make_uint4(0, 0, 0, 0);
  }
  auto value = [&](int i, int e) -> float {
    const uint32_t wd = e < 2 ? raw[i].x : e < 4 ? raw[i].y : e < 6 ? raw[i].z : raw[i].w;
    return (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
  };
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(value(i, e)));
  __shared__ float s_amax[4];
  amax = wave_max_f32(amax);
  if ((t & 63) == 0) s_amax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));
  float s;
  {
#pragma clang fp contract(off)
    const float thr = clip * amax;  // one IEEE fp32 multiply
    s = thr / 127.f;                // IEEE fp32 division (correctly rounded)
  }
  const float rcp = 1.f / s;
  const bool live = s > 0.f;
  int8_t* dst = codes + (size_t)r0 * cols + kb * 128 + cg * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rl + 16 * i;
    if (r < nr) {
      int c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = live ? quant_code(value(i, e), s, rcp) : 0;
      uint2 o;
      o.x = pack4_i8(c[0], c[1], c[2], c[3]);
      o.y = pack4_i8(c[4], c[5], c[6], c[7]);
      *(uint2*)(dst + (size_t)r * cols) = o;
    }
  }
  if (t == 0) scales[(size_t)mb * (cols / 128) + kb] = live ? s : 0.f;
}

// ---------------------------------------------------------------------------------------------------------
// k5_gemm: one workgroup per 128 (tokens) × 256 (outputs) tile of Y, 512 threads (8 waves, 2 per SIMD). Wave
// w owns tokens 64 (w % 2) .. +63 and outputs 64 (w / 2) .. +63 as 2 × 2 MFMA tiles of D = W X^T (32 outputs
// × 32 tokens): each lane then holds one token and runs of 4 consecutive outputs, which it stores as 8 bytes.
// Per k-block (128 input features) the X and W codes of the tile arrive by direct-to-LDS buffer loads in a
// three-slot ring, issued two k-blocks ahead: rows of 128 bytes with their 16-byte chunks XOR-swizzled by
// bits 1..3 of the row, so that the 16 lanes of each LDS read phase (rows r .. r+15 at one chunk) hit 16
// distinct 16-byte bank groups. The four k-steps of the k-block run into int32 accumulators that start at
// zero; each finished partial (exact: |P| <= 127^2 * 128 < 2^24) is folded into the fp32 sums while other
// MFMAs run (see kblock below).
// Rows of X past M (last token tile) and rows of W past N (last output tile when N % 256 == 128) re-read the
// last valid row; their results are never stored.
// ---------------------------------------------------------------------------------------------------------
constexpr int kWThreads = 512;
constexpr int kWTileM = 128, kWTileN = 256;
constexpr int kWMaxKb = 256;  // K <= 32768
constexpr int kWXBytes = kWTileM * 128, kWSlot = kWXBytes + kWTileN * 128;

template <int N>
__device__ __forceinline__ void w_ring_sync() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4));  // vmcnt(N), lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int w_swz(int row) { return (row >> 1) & 7; }

__global__ __launch_bounds__(kWThreads, 1) void k5_gemm(const int8_t* __restrict__ x8, const float* __restrict__ xs,
                                                        const int8_t* __restrict__ w8, const float* __restrict__ ws,
                                                        const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
                                                        int M, int N, int K, int n_mt, int n_nt) {
  // ring slots: X codes at [0, 16 KB), W codes at [16 KB, 48 KB) of each (one LDS object per slot, so that every
  // operand read of a slot is one lane register plus an immediate offset)
  __shared__ __attribute__((aligned(1024))) unsigned char s_r0[kWSlot], s_r1[kWSlot], s_r2[kWSlot];
  __shared__ float s_c[2][kWMaxKb];  // per k-block scale products of the tile's two output blocks

  const int nkb = K >> 7;
  // tile order: XCD-aware, then token tiles in groups of 8 with the output tiles of a group in sequence, so
  // that the workgroups running together on one XCD share both X and W rows in its L2
  const int total = n_mt * n_nt;
  const int f = xcd_remap((int)blockIdx.x, total);
  constexpr int kGroup = 8;
  const int grp = f / (kGroup * n_nt), in_grp = f - grp * kGroup * n_nt;
  const int g_rows = min(kGroup, n_mt - grp * kGroup);
  const int mt = grp * kGroup + in_grp % g_rows, nt = in_grp / g_rows;
  const int m0 = mt * kWTileM, n0 = nt * kWTileN;
  const int mv = min(kWTileM, M - m0), nvld = min(kWTileN, N - n0);

  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int lr = l & 31, g = l >> 5;

  // scale products c[j][kb] = fp32(s_x(mt, kb) * s_w(nb_j, kb)) for the tile's output blocks j = 0, 1
  for (int i = t; i < 2 * nkb; i += kWThreads) {
    const int j = i / nkb, kb = i - j * nkb;
    const int nb = min((n0 >> 7) + j, (N >> 7) - 1);
    s_c[j][kb] = xs[(size_t)mt * nkb + kb] * ws[(size_t)nb * nkb + kb];
  }

  // direct-to-LDS loads: a wave's load fills 1 KB = 8 rows of 128 bytes at LDS chunk positions 64 q + l; lane l
  // takes row 8 q + l / 8 of the tile, chunk (l % 8) ^ swz(row) of the k-block. The lane part of the offset is
  // the same for every k-block; the k-block offset goes in the scalar offset.
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(x8 + (size_t)m0 * K),
                                                                      (short)0, mv * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(w8 + (size_t)n0 * K),
                                                                      (short)0, nvld * K, 0x00020000);
  uint32_t xo[2], wo[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = 8 * i + w, row = 8 * q + (l >> 3);
    xo[i] = (uint32_t)(min(row, mv - 1) * K + 16 * ((l & 7) ^ w_swz(row)));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 8 * i + w, row = 8 * q + (l >> 3);
    wo[i] = (uint32_t)(min(row, nvld - 1) * K + 16 * ((l & 7) ^ w_swz(row)));
  }
  auto stage = [&](int kb, unsigned char* __restrict__ slot) {
    const uint32_t koff = (uint32_t)kb * 128u;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (w_lds_void*)(slot + (8 * i + w) * 1024), 16, xo[i], koff, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w_lds_void*)(slot + kWXBytes + (8 * i + w) * 1024), 16, wo[i],
                                               koff, 0, 0);
  };

  // operand reads: tile row 32 tt + lr, chunk 2 ks + g of the k-block; (row >> 1) & 7 = (lr >> 1) & 7. The lane
  // offsets of this wave's X rows (xr) and W rows (wr) per k-step are loop-invariant; the 32-row tile steps are
  // immediates.
  const int wm = w & 1, wn = w >> 1;
  const int xrow0 = 64 * wm, wrow0 = 64 * wn;
  uint32_t xr[4], wr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t ro = (uint32_t)(lr * 128 + 16 * ((2 * ks + g) ^ ((lr >> 1) & 7)));
    xr[ks] = ro + xrow0 * 128;
    wr[ks] = ro + kWXBytes + wrow0 * 128;
  }
  const int cj_blk = wn >> 1;  // which of the tile's two output blocks this wave's outputs lie in

  v16f acc[2][2];  // fp32 sums [output tile j][token tile i]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (v16f){};
  // int32 partials of two tiles: quarter q of a k-block writes part[q & 1]. part[1] starts at zero so that the
  // first k-block's fold of "the previous quarter 3" adds exactly nothing (c_prev = 0).
  v16i part[2];
  part[1] = (v16i){};

  // One k-block in four quarters, one 32 × 32 tile (j, i) = (q / 2, q % 2) each: its 4 k-steps back to back
  // (the accumulator is forwarded from MFMA to MFMA), each k-step slot also folding a quarter of the previous
  // quarter's partial into its fp32 sums (the fold of quarter 3 runs in the next k-block's quarter 0, with the
  // scale product c_prev of that k-block). Scheduling barriers keep this slot structure, so that only two
  // partial tiles are live and every fold overlaps MFMAs.
  auto kblock = [&](int kb, const unsigned char* __restrict__ slot, float c_prev) {
    // the slot's base plus an offset the compiler cannot see through (always 0): the eight operand addresses
    // are then formed here, once per k-block, instead of being held for every slot across the loop
    int z = 0;
    asm volatile("" : "+s"(z));
    const unsigned char* sb = slot + z;
    const float c = s_c[cj_blk][kb];
    v4i b[4][2], a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      a[ks] = *(const v4i*)(sb + wr[ks]);
#pragma unroll
      for (int i = 0; i < 2; ++i) b[ks][i] = *(const v4i*)(sb + xr[ks] + 4096 * i);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = q & 1;
      const int pq = (q + 3) & 3;  // the previous quarter's tile
      v16f& dst = acc[pq >> 1][pq & 1];
      const v16i& src = part[pq & 1];
      const float cf = q == 0 ? c_prev : c;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        part[q & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ks], b[ks][i], ks == 0 ? (v16i){} : part[q & 1], 0,
                                                             0, 0);
        // after its last use by output tile 0, a[ks] takes output tile 1's fragment
        if (q == 1) a[ks] = *(const v4i*)(sb + wr[ks] + 4096);
#pragma unroll
        for (int r = 4 * ks; r < 4 * ks + 4; ++r) dst[r] = fmaf((float)src[r], cf, dst[r]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: k-blocks 0 and 1. Every iteration issues exactly one stage (six loads per wave), so one wait count
  // fits all of them; past the end a stage re-loads the last k-block into the free slot (in bounds, never read).
  stage(0, s_r0);
  stage(min(1, nkb - 1), s_r1);

  // iteration kb: wait for k-block kb (k-block kb+1 may stay in flight), refill the slot of kb-1 with kb+2, run kb
  auto iter = [&](int kb, const unsigned char* cur, unsigned char* fill) {
    w_ring_sync<6>();
    stage(min(kb + 2, nkb - 1), fill);
    const float cp = s_c[cj_blk][max(kb - 1, 0)];
    kblock(kb, cur, kb > 0 ? cp : 0.f);
  };
  int kb = 0;
  for (; kb + 3 <= nkb; kb += 3) {
    iter(kb + 0, s_r0, s_r2);
    iter(kb + 1, s_r1, s_r0);
    iter(kb + 2, s_r2, s_r1);
  }
  if (kb < nkb) iter(kb, s_r0, s_r2);
  if (kb + 1 < nkb) iter(kb + 1, s_r1, s_r0);
  w_ring_sync<0>();  // the trailing re-loads have landed before the workgroup's LDS can be handed on
  {
    const float c = s_c[cj_blk][nkb - 1];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[1][1][r] = fmaf((float)part[1][r], c, acc[1][1][r]);
  }

  // store: acc[j][i][r] = Y[token m0 + xrow0 + 32 i + lr][output n0 + wrow0 + 32 j + 8 (r / 4) + 4 g + r % 4]
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = xrow0 + 32 * i + lr;
    if (m >= mv) continue;
    uint16_t* yrow = y + (size_t)(m0 + m) * N + n0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = wrow0 + 32 * j + 8 * q + 4 * g;
        if (n >= nvld) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[j][i][4 * q + e];
        if (bias) {
          const uint2 b = *(const uint2*)(bias + n0 + n);
          v[0] += bf16_lo(b.x);
          v[1] += bf16_hi(b.x);
          v[2] += bf16_lo(b.y);
          v[3] += bf16_hi(b.y);
        }
        *(uint2*)(yrow + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
  }
}

hipError_t launch_w8a8_quant(const uint16_t* x, int rows, int cols, float clip, int8_t* codes, float* scales,
                             hipStream_t s) {
  hipLaunchKernelGGL(k5_quant, dim3(cols / 128, (rows + 127) / 128), dim3(256), 0, s, x, rows, cols, clip, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_w8a8_gemm(const int8_t* x8, const float* xs, const int8_t* w8, const float* ws,
                            const uint16_t* bias, uint16_t* y, int M, int N, int K, hipStream_t s) {
  const int n_mt = (M + kWTileM - 1) / kWTileM, n_nt = (N + kWTileN - 1) / kWTileN;
  hipLaunchKernelGGL(k5_gemm, dim3(n_mt * n_nt), dim3(kWThreads), 0, s, x8, xs, w8, ws, bias, y, M, N, K, n_mt,
                     n_nt);
  return hipGetLastError();
}

}  // namespace sagesla
