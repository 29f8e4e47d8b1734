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
// k5_gemm: one workgroup per 256 (tokens) × 256 (outputs) tile of Y, 512 threads (8 waves, 2 per SIMD). Wave
// w owns tokens 64 (w % 4) .. +63 and outputs 128 (w / 4) .. +127 -- one 128-token block and one 128-output
// block, so one scale product per k-block -- as 2 × 4 MFMA tiles of D = W X^T (32 outputs × 32 tokens): each
// lane then holds one token and runs of 4 consecutive outputs, which it stores as 8 bytes.
// Per k-block (128 input features) the X and W codes of the tile arrive by direct-to-LDS buffer loads in a
// two-slot ring (64 KB a slot), the next k-block's loads landing while this one is computed: rows of 128 bytes
// with their 16-byte chunks XOR-swizzled by bits 1..3 of the row, so that the 16 lanes of each LDS read phase
// (rows r .. r+15 at one chunk) hit 16 distinct 16-byte bank groups. The tile size sets the load traffic per
// MFMA: every byte brought in feeds 256 multiply-adds, which the per-CU load path sustains.
// Each 32 × 32 tile's four k-steps run into int32 accumulators that start at zero; each finished partial
// (exact: |P| <= 127^2 * 128 < 2^24) is folded into the fp32 sums while the next tile's MFMAs run.
// Rows of X past M (last token tile) and rows of W past N (last output tile when N % 256 == 128) re-read the
// last valid row; their results are never stored.
// ---------------------------------------------------------------------------------------------------------
constexpr int kWThreads = 512;
constexpr int kWTile = 256;   // tokens and outputs per workgroup tile
constexpr int kWMaxKb = 256;  // K <= 32768
constexpr int kWXBytes = kWTile * 128, kWSlot = 2 * kWXBytes;

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
  // ring slots: X codes at [0, 32 KB), W codes at [32 KB, 64 KB) of each (one LDS object per slot, so that every
  // operand read of a slot is one lane register plus an immediate offset)
  __shared__ __attribute__((aligned(1024))) unsigned char s_r0[kWSlot], s_r1[kWSlot];
  __shared__ float s_c[2][2][kWMaxKb];  // scale products [token block][output block][k-block] of the tile

  const int nkb = K >> 7;
  // tile order: XCD-aware, then token tiles in groups of 8 with the output tiles of a group in sequence, so
  // that the workgroups running together on one XCD share both X and W rows in its L2
  const int total = n_mt * n_nt;
  const int f = xcd_remap((int)blockIdx.x, total);
  constexpr int kGroup = 8;
  const int grp = f / (kGroup * n_nt), in_grp = f - grp * kGroup * n_nt;
  const int g_rows = min(kGroup, n_mt - grp * kGroup);
  const int mt = grp * kGroup + in_grp % g_rows, nt = in_grp / g_rows;
  const int m0 = mt * kWTile, n0 = nt * kWTile;
  const int mv = min(kWTile, M - m0), nvld = min(kWTile, N - n0);

  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int lr = l & 31, g = l >> 5;

  // scale products c[a][b][kb] = fp32(s_x(mb_a, kb) * s_w(nb_b, kb)) for the tile's token blocks a and output
  // blocks b (blocks past the end are clamped; their results are never stored)
  {
    const int n_mblk = (M + 127) >> 7, n_nblk = N >> 7;
    for (int i = t; i < 4 * nkb; i += kWThreads) {
      const int ab = i / nkb, kb = i - ab * nkb;
      const int mb = min((m0 >> 7) + (ab >> 1), n_mblk - 1), nb = min((n0 >> 7) + (ab & 1), n_nblk - 1);
      s_c[ab >> 1][ab & 1][kb] = xs[(size_t)mb * nkb + kb] * ws[(size_t)nb * nkb + kb];
    }
  }

  // direct-to-LDS loads: a wave's load fills 1 KB = 8 rows of 128 bytes at LDS chunk positions 64 q + l; lane l
  // takes row 8 q + l / 8 of the tile, chunk (l % 8) ^ swz(row) of the k-block. The lane part of the offset is
  // the same for every k-block; the k-block offset goes in the scalar offset.
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(x8 + (size_t)m0 * K),
                                                                      (short)0, mv * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(w8 + (size_t)n0 * K),
                                                                      (short)0, nvld * K, 0x00020000);
  uint32_t xo[4], wo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 8 * i + w, row = 8 * q + (l >> 3);
    const uint32_t ch = 16 * ((l & 7) ^ w_swz(row));
    xo[i] = (uint32_t)(min(row, mv - 1) * K) + ch;
    wo[i] = (uint32_t)(min(row, nvld - 1) * K) + ch;
  }
  auto stage = [&](int kb, unsigned char* __restrict__ slot) {
    const uint32_t koff = (uint32_t)kb * 128u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (w_lds_void*)(slot + (8 * i + w) * 1024), 16, xo[i], koff, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (w_lds_void*)(slot + kWXBytes + (8 * i + w) * 1024), 16, wo[i],
                                               koff, 0, 0);
  };

  // operand reads: tile row 32 tt + lr, chunk 2 ks + g of the k-block; (row >> 1) & 7 = (lr >> 1) & 7. The lane
  // offsets of this wave's X rows (xr) and W rows (wr) per k-step are loop-invariant; the 32-row tile steps are
  // immediates.
  const int wm = w & 3, wn = w >> 2;
  const int xrow0 = 64 * wm, wrow0 = 128 * wn;
  uint32_t xr[4], wr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t ro = (uint32_t)(lr * 128 + 16 * ((2 * ks + g) ^ ((lr >> 1) & 7)));
    xr[ks] = ro + xrow0 * 128;
    wr[ks] = ro + kWXBytes + wrow0 * 128;
  }
  const int cm = wm >> 1, cn = wn;  // this wave's token block and output block inside the tile

  v16f acc[4][2];  // fp32 sums [output tile j][token tile i]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (v16f){};
  // int32 partials of two tiles: tile u = 2 j + i of a k-block writes part[u & 1]. Both start at zero so that the
  // first k-block's folds of "the previous k-block's tiles 6 and 7" add exactly nothing (c_prev = 0).
  v16i part[2];
  part[0] = (v16i){};
  part[1] = (v16i){};

  // One k-block as eight tiles u = 2 j + i, each with its 4 k-steps back to back (the accumulator is forwarded
  // from MFMA to MFMA). The previous tile's partial is folded into its fp32 sums one MFMA late, so that its last
  // MFMA has finished: k-step slots 1-3 of tile u fold elements 0-11 of tile u-1 after their MFMA, and slot 0 of
  // tile u+1 folds its elements 12-15 before its own MFMA takes the registers. Tiles 6 and 7 are completed in the
  // next k-block with that k-block's scale product c_prev. The W fragments of output tile j + 1 replace those of
  // tile j right after their last use. Scheduling barriers keep this slot structure, so that only two partial
  // tiles are live and no fold waits for an MFMA.
  auto fold4 = [&](int v, int r0, float cf) {
    v16f& dst = acc[v >> 1][v & 1];
    const v16i& src = part[v & 1];
#pragma unroll
    for (int r = r0; r < r0 + 4; ++r) dst[r] = fmaf((float)src[r], cf, dst[r]);
  };
  auto kblock = [&](int kb, const unsigned char* __restrict__ slot, float c_prev) {
    // the slot's base plus an offset the compiler cannot see through (always 0): the eight operand addresses
    // are then formed here, once per k-block, instead of being held for every slot across the loop
    int z = 0;
    asm volatile("" : "+s"(z));
    const unsigned char* sb = slot + z;
    const float c = s_c[cm][cn][kb];
    v4i b[4][2], a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      a[ks] = *(const v4i*)(sb + wr[ks]);
#pragma unroll
      for (int i = 0; i < 2; ++i) b[ks][i] = *(const v4i*)(sb + xr[ks] + 4096 * i);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = u >> 1, i = u & 1;
      const int u1 = (u + 7) & 7, u2 = (u + 6) & 7;    // the two previous tiles (of this or the last k-block)
      const float c1 = u >= 1 ? c : c_prev, c2 = u >= 2 ? c : c_prev;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 0) fold4(u2, 12, c2);  // reads part[u & 1] before this tile's first MFMA overwrites it
        part[u & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ks], b[ks][i], ks == 0 ? (v16i){} : part[u & 1], 0,
                                                             0, 0);
        if (i == 1 && j < 3) a[ks] = *(const v4i*)(sb + wr[ks] + 4096 * (j + 1));
        if (ks >= 1) fold4(u1, 4 * (ks - 1), c1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Two-slot ring: iteration kb waits for k-block kb (the only load in flight), then refills the other slot
  // (read in iteration kb - 1, which every wave has finished) with k-block kb + 1, then computes kb. Every
  // iteration issues exactly one stage, so one wait count fits all; past the end a stage re-loads the last
  // k-block (in bounds, never read).
  stage(0, s_r0);
  auto iter = [&](int kb, const unsigned char* cur, unsigned char* fill) {
    w_ring_sync<0>();
    stage(min(kb + 1, nkb - 1), fill);
    const float cp = s_c[cm][cn][max(kb - 1, 0)];
    kblock(kb, cur, kb > 0 ? cp : 0.f);
  };
  int kb = 0;
  for (; kb + 2 <= nkb; kb += 2) {
    iter(kb + 0, s_r0, s_r1);
    iter(kb + 1, s_r1, s_r0);
  }
  if (kb < nkb) iter(kb, s_r0, s_r1);
  w_ring_sync<0>();  // the trailing re-load has landed before the workgroup's LDS can be handed on
  {
    const float c = s_c[cm][cn][nkb - 1];  // the last k-block's tiles 6 (elements 12-15) and 7 (all)
    fold4(6, 12, c);
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += 4) fold4(7, r0, c);
  }

  // store: acc[j][i][r] = Y[token m0 + xrow0 + 32 i + lr][output n0 + wrow0 + 32 j + 8 (r / 4) + 4 g + r % 4]
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = xrow0 + 32 * i + lr;
    if (m >= mv) continue;
    uint16_t* yrow = y + (size_t)(m0 + m) * N + n0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = wrow0 + 32 * j + 8 * q + 4 * g;
        if (n >= nvld) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[j][i][4 * q + e];
        if (bias) {
          const uint2 bb = *(const uint2*)(bias + n0 + n);
          v[0] += bf16_lo(bb.x);
          v[1] += bf16_hi(bb.x);
          v[2] += bf16_lo(bb.y);
          v[3] += bf16_hi(bb.y);
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
  const int n_mt = (M + kWTile - 1) / kWTile, n_nt = (N + kWTile - 1) / kWTile;
  hipLaunchKernelGGL(k5_gemm, dim3(n_mt * n_nt), dim3(kWThreads), 0, s, x8, xs, w8, ws, bias, y, M, N, K, n_mt,
                     n_nt);
  return hipGetLastError();
}

}  // namespace sagesla
