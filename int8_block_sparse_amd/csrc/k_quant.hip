// K1: K-mean smoothing, per-block INT8 quantization and block mean pooling (gfx950).
//
// "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn), §三(一) SageAttention2++: item 1 smooths
// outliers before quantizing, item 2 gives every sub-block its own quantization parameters. Here:
//   mu[c]   = fp32(exact sum over all N tokens of K[t][c] / N)     (per (b, h) channel mean of K)
//   k'      = fp32(K - mu)                                          (Q and V are not smoothed)
//   scale   = fp32(absmax / 127) per block of rows × all D channels (0 for an all-zero block), or per 32 rows
//             (the pages' thread-level granularity, §三(一) item 2)
//   code    = clamp(round-half-even(fp32(x / scale)), -127, 127)
//   pool    = fp64 mean of the block's rows (raw Q; smoothed K)
// The fp64 column sums are exact when every partial sum is representable, which holds for bf16 inputs whose
// sum of magnitudes stays below 2^53 units of the smallest ulp; the result is then independent of order.
// HBM bound: K is read twice (sum, then quantize), Q once; int8 codes are written once.
#include "device_common.h"
#include "internal.h"
#include "lin_common.h"

namespace sagesla {

// K0: RMSNorm of Q and K over all H*D channels of each token. grid (ceil(N / 8), B, 2: Q then K), 512 threads:
// wave w takes token 8 blockIdx.x + w; lane l holds channels 8 (l % 16) .. +7 of heads 4 i + l / 16, so one
// 16-byte load per lane covers four whole 256-byte head rows, and all of a token's loads are in flight at once
// (up to 64 heads held in registers; more heads are read again for the output). The sum of squares (each square
// of a bf16 value is exact in fp64) is kept as a double-double (Knuth's error-free TwoSum) per lane and through
// the lane-exchange tree, so it is within n^2 2^-106 of the exact sum before its single rounding to fp64; TwoSum
// is symmetric in its operands, so every lane of the tree ends with the same value. Output:
// x_hat = bf16(fp32(bf16(fp32(x * r)) * w)).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

constexpr int kNormRegLoads = 16;  // head groups of 4 kept in registers (H <= 64)

__global__ __launch_bounds__(512) void k0_rmsnorm(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
                                                  uint16_t* __restrict__ q_hat, uint16_t* __restrict__ k_hat, int H,
                                                  int N, float eps) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int n = blockIdx.x * 8 + w, b = blockIdx.y;
  if (n >= N) return;  // whole wave: no barrier in this kernel
  const bool isk = blockIdx.z != 0;
  const uint16_t* src = isk ? k : q;
  const uint16_t* wt = isk ? wk : wq;
  uint16_t* dst = isk ? k_hat : q_hat;
  const int hs = l >> 4, c0 = 8 * (l & 15);
  const size_t plane = (size_t)N * kD;  // elements per (b, h) plane
  const size_t base = (size_t)b * H * plane + (size_t)n * kD + c0;
  const int ng = (H + 3) >> 2;  // head groups of 4
  auto row = [&](int i) { return base + (size_t)(4 * i + hs) * plane; };
  auto live = [&](int i) { return 4 * i + hs < H; };

  uint4 x[kNormRegLoads];
#pragma unroll
  for (int i = 0; i < kNormRegLoads; ++i)
    x[i] = (i < ng && live(i)) ? *(const uint4*)(src + row(i)) : make_uint4(0, 0, 0, 0);
  double hi = 0.0, lo = 0.0, e;
  auto acc8 = [&](const uint4& v) {
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double a = (double)bf16_lo(wd[j]), c = (double)bf16_hi(wd[j]);
      two_sum(hi, a * a, hi, e);
      lo += e;
      two_sum(hi, c * c, hi, e);
      lo += e;
    }
  };
#pragma unroll
  for (int i = 0; i < kNormRegLoads; ++i)
    if (i < ng) acc8(x[i]);
  for (int i = kNormRegLoads; i < ng; ++i)
    if (live(i)) acc8(*(const uint4*)(src + row(i)));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double ho = __shfl_xor(hi, o), lw = __shfl_xor(lo, o);
    two_sum(hi, ho, hi, e);
    lo = (lo + lw) + e;
  }
  const double m = (hi + lo) / (double)(H * kD);
  const float r = (float)(1.0 / sqrt(m + (double)eps));
  auto norm8 = [&](int i, const uint4& v) {
    const int h = 4 * i + hs;
    const uint4 g = *(const uint4*)(wt + h * kD + c0);
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float n0, n1, y0, y1;
      {
#pragma clang fp contract(off)
        n0 = bf16_lo(wd[j]) * r;
        n1 = bf16_hi(wd[j]) * r;
      }
      const uint32_t nb = pack_bf16x2(n0, n1);
      {
#pragma clang fp contract(off)
        y0 = bf16_lo(nb) * bf16_lo(gw[j]);
        y1 = bf16_hi(nb) * bf16_hi(gw[j]);
      }
      o[j] = pack_bf16x2(y0, y1);
    }
    *(uint4*)(dst + row(i)) = make_uint4(o[0], o[1], o[2], o[3]);
  };
#pragma unroll
  for (int i = 0; i < kNormRegLoads; ++i)
    if (i < ng && live(i)) norm8(i, x[i]);
  for (int i = kNormRegLoads; i < ng; ++i)
    if (live(i)) norm8(i, *(const uint4*)(src + row(i)));
}

// Partial column sums of K over row chunks, fp64. grid (n_chunks, BH), 256 threads:
// thread t reads channels 8*(t%16)..+7 of rows t/16, t/16+16, ... (a wave reads 4 whole rows per load).
__global__ __launch_bounds__(256) void k1_colsum_partial(const uint16_t* __restrict__ k, double* __restrict__ part,
                                                        int N, int chunk_rows, int n_chunks) {
  const int bh = blockIdx.y, ch = blockIdx.x;
  const int t = threadIdx.x, cg = t & 15, rl = t >> 4;
  const uint16_t* base = k + (size_t)bh * N * kD + cg * 8;
  const int r0 = ch * chunk_rows, r1 = min(N, r0 + chunk_rows);
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  int r = r0 + rl;
  for (; r + 48 < r1; r += 64) {
    uint4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = *(const uint4*)(base + (size_t)(r + 16 * u) * kD);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[0] += bf16_lo(w[u].x); acc[1] += bf16_hi(w[u].x);
      acc[2] += bf16_lo(w[u].y); acc[3] += bf16_hi(w[u].y);
      acc[4] += bf16_lo(w[u].z); acc[5] += bf16_hi(w[u].z);
      acc[6] += bf16_lo(w[u].w); acc[7] += bf16_hi(w[u].w);
    }
  }
  for (; r < r1; r += 16) {
    uint4 w = *(const uint4*)(base + (size_t)r * kD);
    acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
    acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
    acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
    acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
  }
  __shared__ double red[16][kD + 1];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rl][cg * 8 + i] = acc[i];
  __syncthreads();
  if (t < kD) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += red[j][t];
    part[((size_t)bh * n_chunks + ch) * kD + t] = s;
  }
}

// mu = fp32(S / N), S = the partial sums added in chunk order. grid BH, 128 threads.
__global__ __launch_bounds__(128) void k1_colsum_final(const double* __restrict__ part, float* __restrict__ mu,
                                                      int n_chunks, int N) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const double* p = part + (size_t)bh * n_chunks * kD + c;
  double s = 0.0;
  int i = 0;
  for (; i + 8 <= n_chunks; i += 8) {  // eight loads in flight, added in chunk order
    double x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = p[(size_t)(i + u) * kD];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += x[u];
  }
  for (; i < n_chunks; ++i) s += p[(size_t)i * kD];
  mu[bh * kD + c] = (float)(s / (double)N);
}

// One block of up to MAXROWS rows (valid: `rows`) × 128 channels, 256 threads. Thread t owns channels
// 8*(t%16)..+7 of rows t/16 + 16*i.
// One block of rows (<= MAXROWS) of D channels: thread (row group rl, 8-channel group cg) holds rows rl + 16 i.
// Rows stay packed bf16 in registers (4 words per 8 values); with SMOOTH the fp32 value k - mu is formed again
// where it is needed (the same single IEEE subtraction each time).
// With G32 the block's rows get one scale per 32 rows (group g = rows 32 g .. +31 = the rows of steps i = 2g, 2g+1
// of every thread); scale_out then receives one value per group that holds a valid row.
// With kt_img (key blocks of 64 rows only) the block's raw rows also go to LDS as a K^T image in the V^T-image
// layout (write_v_image below: channel rows of 64 key slots, zeros past `rows`), for the linear-branch state.
// With norm_out (key blocks only) each scale's rows also give the largest squared Euclidean norm of their codes
// (exact in int32), in norm_out's slot for that scale: the attention kernel bounds its scores with it.
template <int MAXROWS, bool SMOOTH, bool G32>
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ src, int rows, const float* __restrict__ mu,
                                            int8_t* __restrict__ dst, float* __restrict__ scale_out,
                                            double* __restrict__ pool_out, float (*s_amax)[4],
                                            double (*s_red)[kD + 1], unsigned char* __restrict__ kt_img = nullptr,
                                            int32_t* __restrict__ norm_out = nullptr, int (*s_kn)[4] = nullptr) {
  constexpr int IT = MAXROWS / 16;
  constexpr int NG = G32 ? MAXROWS / 32 : 1;  // scales in this block
  const int t = threadIdx.x, cg = t & 15, rl = t >> 4;
  float m8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m8[e] = SMOOTH ? mu[cg * 8 + e] : 0.f;
  uint4 raw[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int r = rl + 16 * i;
    raw[i] = (r < rows) ? *(const uint4*)(src + (size_t)r * kD + cg * 8) : make_uint4(0, 0, 0, 0);
  }
  if constexpr (MAXROWS == kBlkK) {
    if (kt_img) {  // row rl + 16 i is key slot 16 i + key_pos16(rl) of channel rows 8 cg .. +7
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const int pos = 16 * i + key_pos16(rl);
        const uint32_t wd[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int row = cg * 8 + e;
          *(uint16_t*)(kt_img + row * 128 + (((pos >> 3) ^ swz32(row)) << 4) + ((pos & 7) << 1)) =
              (uint16_t)((e & 1) ? wd[e >> 1] >> 16 : wd[e >> 1] & 0xffffu);
        }
      }
    }
  }
  auto value = [&](int i, int e) -> float {  // element e of row rl + 16 i, smoothed when SMOOTH (0 past rows)
    const uint32_t wd = e < 2 ? raw[i].x : e < 4 ? raw[i].y : e < 6 ? raw[i].z : raw[i].w;
    const float x = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
    return SMOOTH ? (rl + 16 * i < rows ? x - m8[e] : 0.f) : x;  // one IEEE fp32 subtraction
  };
  float amax[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) amax[gi] = 0.f;
  double psum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) psum[e] = 0.0;
#pragma unroll
  for (int i = 0; i < IT; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = value(i, e);
      amax[G32 ? i / 2 : 0] = fmaxf(amax[G32 ? i / 2 : 0], fabsf(x));
      psum[e] += (double)x;
    }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    amax[gi] = wave_max_f32(amax[gi]);
    if ((t & 63) == 0) s_amax[t >> 6][gi] = amax[gi];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_red[rl][cg * 8 + e] = psum[e];
  __syncthreads();
  float s[NG], rcp[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    amax[gi] = fmaxf(fmaxf(s_amax[0][gi], s_amax[1][gi]), fmaxf(s_amax[2][gi], s_amax[3][gi]));
    s[gi] = amax[gi] / 127.f;  // IEEE fp32 division (correctly rounded)
    rcp[gi] = 1.f / s[gi];
  }
  int n2[IT];  // squared norm of this thread's 8 codes of row rl + 16 i (0 past the valid rows)
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int r = rl + 16 * i, gi = G32 ? i / 2 : 0;
    n2[i] = 0;
    if (r < rows) {
      int c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = (amax[gi] > 0.f) ? quant_code(value(i, e), s[gi], rcp[gi]) : 0;
      uint2 o;
      o.x = pack4_i8(c[0], c[1], c[2], c[3]);
      o.y = pack4_i8(c[4], c[5], c[6], c[7]);
      *(uint2*)(dst + (size_t)r * kD + cg * 8) = o;
#pragma unroll
      for (int e = 0; e < 8; ++e) n2[i] += c[e] * c[e];
    }
  }
  if constexpr (MAXROWS == kBlkK) {
    if (norm_out) {  // a row's 16 threads are lanes 16 k .. 16 k + 15 of one wave
      int nm[NG];
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) nm[gi] = 0;
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        int v = n2[i];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
        nm[G32 ? i / 2 : 0] = max(nm[G32 ? i / 2 : 0], v);
      }
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        nm[gi] = max(nm[gi], __shfl_xor(nm[gi], 16));
        nm[gi] = max(nm[gi], __shfl_xor(nm[gi], 32));
        if ((t & 63) == 0) s_kn[t >> 6][gi] = nm[gi];
      }
      __syncthreads();
      if (t < NG && 32 * t < rows) norm_out[t] = max(max(s_kn[0][t], s_kn[1][t]), max(s_kn[2][t], s_kn[3][t]));
    }
  }
  if (t < kD) {
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += s_red[j][t];
    pool_out[t] = sum / (double)rows;
  }
  if (t < NG && 32 * t < rows) scale_out[t] = (amax[t] > 0.f) ? s[t] : 0.f;
}

// rows of one key block of V as the V^T image writer takes them: thread (cg, kg) holds keys 4 kg .. +3,
// channels 8 cg .. +7 (zeros past nv)
__device__ __forceinline__ void load_v_rows(const uint16_t* __restrict__ src, int nv, uint32_t (&wv)[4][4]) {
  const int t = threadIdx.x, cg = t & 15, kg = t >> 4;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int r = 4 * kg + b;
    uint4 a = make_uint4(0, 0, 0, 0);
    if (r < nv) a = *(const uint4*)(src + (size_t)r * kD + cg * 8);
    wv[b][0] = a.x; wv[b][1] = a.y; wv[b][2] = a.z; wv[b][3] = a.w;
  }
}

// V^T image of one key block for the attention kernel: [128 channels][64 keys] bf16, 16 KB, each channel row's
// keys in MFMA slot order (key_pos16 within every 16) and its 16-byte chunks XOR-swizzled (swz32), exactly the
// LDS layout the attention kernel reads; keys past a ragged block's end are zero. 256 threads: thread t holds
// (load_v_rows) channels 8*(t%16)..+7 of keys 4*(t/16)..+3.
__device__ __forceinline__ void write_v_image(const uint32_t (&wv)[4][4], unsigned char* __restrict__ img) {
  const int t = threadIdx.x, cg = t & 15, kg = t >> 4;
  const int pos = 16 * (kg >> 2) + key_pos16(4 * (kg & 3));
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = cg * 8 + e, sh = (e & 1) * 16;
    const uint32_t k0 = (wv[0][e >> 1] >> sh) & 0xffffu, k1 = (wv[1][e >> 1] >> sh) & 0xffffu;
    const uint32_t k2 = (wv[2][e >> 1] >> sh) & 0xffffu, k3 = (wv[3][e >> 1] >> sh) & 0xffffu;
    *(uint2*)(img + row * 128 + (((pos >> 3) ^ swz32(row)) << 4) + ((pos & 7) << 1)) =
        make_uint2(k0 | (k1 << 16), k2 | (k3 << 16));
  }
}

// The forward's linear-branch state of key block J ("Turbo Diffusion", lanhy.cn, §三(二) SLA item 2):
// H_J^T = (phi(K_J)^T V_J)^T (D×D) and Z_J = sum over the block's keys of phi(K_J) (D), phi = elu + 1 on the raw
// bf16 k, formed by the workgroup that has just quantized block J and still holds its V rows in registers (wv).
// K^T and V^T are in LDS in the V^T-image layout: the quantizer wrote K^T from its registers (s_kt), V^T goes to
// the quantizer's reduction buffer once that is free (s_vt). One MFMA operand is a V^T image row (channel e, 8
// key slots), the other phi of a K^T image row (channel c,
// the same key slots) split into bf16 hi + lo, so every product keeps ~16 significant bits; keys past a ragged
// block's end are zero in both images and phi of them is taken as 0 for Z_J. Wave w owns channels c = 32 w ..
// +31, so acc[mt] holds rows e = 32 mt .. +31.
// Stored in fp16 with one power of two per block: with M the largest magnitude over H_J^T and Z_J and k its
// frexp exponent (M < 2^k), x is stored as fp16(x * 2^(15 - k)) and e_J = k - 15 (kExpZero for an all-zero
// block). Table [BH][kStateX / 128][n_kb][128] fp16: column group x < 128 of block J is row x of H_J^T, group 128
// is Z_J, each 256 contiguous bytes.
__device__ __forceinline__ void block_state16(const uint32_t (&wv)[4][4], int nv, unsigned char* __restrict__ s_vt,
                                              const unsigned char* __restrict__ s_kt,
                                              float* __restrict__ s_m, uint16_t* __restrict__ table,
                                              int32_t* __restrict__ bexp, int bh, int J, int n_kb) {
  const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 5, lr = l & 31;
  __syncthreads();  // the quantizer's last reads of the reused LDS are done (and its K^T image is written)
  write_v_image(wv, s_vt);
  __syncthreads();

  const int crow = 32 * w + lr;
  v16f acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = (v16f){};
  float z = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int ch = 2 * s + g;  // image chunk: key slots 16 s + 8 g .. +7
    const uint4 kr = *(const uint4*)(s_kt + crow * 128 + ((ch ^ swz32(crow)) << 4));
    const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
    float pk[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = (j & 1) ? bf16_hi(kw[j >> 1]) : bf16_lo(kw[j >> 1]);
      pk[j] = 16 * s + key_pos16(8 * g + j) < nv ? phi_f(x) : 0.f;  // the slot's key index
      z += pk[j];
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(pk[2 * i], pk[2 * i + 1], hi[i], lo[i]);
    const v8bf bh_ = __builtin_bit_cast(v8bf, make_uint4(hi[0], hi[1], hi[2], hi[3]));
    const v8bf bl_ = __builtin_bit_cast(v8bf, make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int er = 32 * mt + lr;
      const v8bf a = *(const v8bf*)(s_vt + er * 128 + ((ch ^ swz32(er)) << 4));
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh_, acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl_, acc[mt], 0, 0, 0);
    }
  }
  z += swap_halves_f32(z);  // both halves of the wave now hold Z_J[crow]

  // the block's largest magnitude and its exponent
  float m = z;  // z >= 0
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[mt][r]));
  m = wave_max_f32(m);
  if (l == 0) s_m[w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  int kx = 0;
  (void)frexpf(m, &kx);  // m < 2^kx
  const int sh = 15 - kx;
  if (t == 0) bexp[(size_t)bh * n_kb + J] = m > 0.f ? kx - 15 : kExpZero;

  // store: neighbouring columns c, c + 1 of one row go out as one 4-byte word. Lanes c and c ^ 1 trade one value
  // of each register pair (r, r + 1) (rows e, e + 1): the even lane writes row e, the odd lane row e + 1.
  const size_t gstride = (size_t)n_kb * 128;  // halves between column groups
  uint16_t* tb = table + (size_t)bh * (kStateX / 128) * gstride + (size_t)J * 128;
  const bool odd = crow & 1;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float a0 = acc[mt][r], a1 = acc[mt][r + 1];
      const float send = odd ? a0 : a1;
      const float got = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));
      const float x0 = odd ? got : a0, x1 = odd ? a1 : got;
      const int e = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3) + (odd ? 1 : 0);
      *(uint32_t*)(tb + (size_t)e * gstride + (crow & ~1)) = pack_f16x2(ldexpf(x0, sh), ldexpf(x1, sh));
    }
  if (g == 0) tb[(size_t)kD * gstride + crow] = (uint16_t)(pack_f16x2(ldexpf(z, sh), 0.f) & 0xffffu);
}

// grid (n_qb + n_kb, BH): x < n_qb quantizes query block x, otherwise key block x - n_qb (and, when v is given,
// writes that key block's V^T image and, when st16 is given too, its linear-branch state: block_state16).
template <int BLKQ, bool G32>
// four workgroups per CU (at most 128 registers): the state's MFMA accumulators then share the quantizer's VGPRs
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k1_quant(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ mu,
    int8_t* __restrict__ q8, int8_t* __restrict__ k8, float* __restrict__ qs, float* __restrict__ ks,
    double* __restrict__ qp, double* __restrict__ kp, int32_t* __restrict__ kn2, const uint16_t* __restrict__ v,
    unsigned char* __restrict__ v_img, uint16_t* __restrict__ st16, int32_t* __restrict__ st_exp, int N, int n_qb,
    int n_kb) {
  __shared__ float s_amax[4][4];
  __shared__ int s_kn[4][4];
  __shared__ __attribute__((aligned(16))) double s_red[16][kD + 1];  // 16512 B: also the state's V^T image
  __shared__ __attribute__((aligned(16))) unsigned char s_kt[kD * 128];
  const int bh = blockIdx.y;
  const int x = blockIdx.x;
  const size_t base = (size_t)bh * N * kD;
  // scales per block, or per 32 tokens with G32 (n_g = ceil(N / 32) of them per (b, h))
  const int n_g = (N + 31) / 32;
  if (x < n_qb) {
    const int r0 = x * BLKQ;
    float* so = G32 ? qs + (size_t)bh * n_g + x * (BLKQ / 32) : qs + (size_t)bh * n_qb + x;
    quant_block<BLKQ, false, G32>(q + base + (size_t)r0 * kD, min(BLKQ, N - r0), nullptr,
                                  q8 + base + (size_t)r0 * kD, so, qp + ((size_t)bh * n_qb + x) * kD, s_amax, s_red);
  } else {
    const int j = x - n_qb;
    const int r0 = j * kBlkK, nv = min(kBlkK, N - r0);
    const size_t sidx = G32 ? (size_t)bh * n_g + j * (kBlkK / 32) : (size_t)bh * n_kb + j;
    float* so = ks + sidx;
    uint32_t wv[4][4];
    if (v) load_v_rows(v + base + (size_t)r0 * kD, nv, wv);  // in flight while K is quantized
    unsigned char* kt = (v && st16) ? s_kt : nullptr;  // the state's K^T image, written by the quantizer
    if (mu)
      quant_block<kBlkK, true, G32>(k + base + (size_t)r0 * kD, nv, mu + bh * kD, k8 + base + (size_t)r0 * kD, so,
                                    kp + ((size_t)bh * n_kb + j) * kD, s_amax, s_red, kt, kn2 + sidx, s_kn);
    else
      quant_block<kBlkK, false, G32>(k + base + (size_t)r0 * kD, nv, nullptr, k8 + base + (size_t)r0 * kD, so,
                                     kp + ((size_t)bh * n_kb + j) * kD, s_amax, s_red, kt, kn2 + sidx, s_kn);
    if (v) write_v_image(wv, v_img + ((size_t)bh * n_kb + j) * 16384);
    if (kt) block_state16(wv, nv, (unsigned char*)&s_red[0][0], s_kt, &s_amax[0][0], st16, st_exp, bh, j, n_kb);
  }
}

__global__ void k_fill_f32(float* __restrict__ d, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) d[i] = v;
}

hipError_t launch_fill_f32(float* dst, size_t n, float val, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)blocks), dim3(256), 0, s, dst, n, val);
  return hipGetLastError();
}

hipError_t launch_qk_norm(const Plan& p, const uint16_t* q, const uint16_t* k, hipStream_t s) {
  hipLaunchKernelGGL(k0_rmsnorm, dim3((p.N + 7) / 8, p.B, 2), dim3(512), 0, s, q, k, (const uint16_t*)p.q_norm_w,
                     (const uint16_t*)p.k_norm_w, p.q_hat, p.k_hat, p.H, p.N, p.norm_eps);
  return hipGetLastError();
}

hipError_t launch_kmean(const Plan& p, const uint16_t* k, hipStream_t s) {
  if (!p.smooth) return launch_fill_f32(p.k_mean, (size_t)p.BH * kD, 0.f, s);
  hipLaunchKernelGGL(k1_colsum_partial, dim3(p.n_colsum_chunks, p.BH), dim3(256), 0, s, k, p.colsum_part, p.N,
                     p.colsum_chunk, p.n_colsum_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k1_colsum_final, dim3(p.BH), dim3(kD), 0, s, p.colsum_part, p.k_mean, p.n_colsum_chunks, p.N);
  return hipGetLastError();
}

hipError_t launch_quant(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v, hipStream_t s) {
  const dim3 grid(p.n_qb + p.n_kb, p.BH);
  const float* mu = p.smooth ? p.k_mean : nullptr;
  uint16_t* st16 = p.states_in_quant ? p.state16 : nullptr;  // the forward's linear-branch state table
#define SAGESLA_QUANT(BQ, G)                                                                                   \
  hipLaunchKernelGGL((k1_quant<BQ, G>), grid, dim3(256), 0, s, q, k, mu, p.q_i8, p.k_i8, p.q_scale, p.k_scale,     \
                     p.q_pool, p.k_pool, p.k_norm2, v, p.v_img, st16, p.state_exp, p.N, p.n_qb, p.n_kb)
  if (p.blk_q == 128) {
    if (p.group32) SAGESLA_QUANT(128, true); else SAGESLA_QUANT(128, false);
  } else {
    if (p.group32) SAGESLA_QUANT(64, true); else SAGESLA_QUANT(64, false);
  }
#undef SAGESLA_QUANT
  return hipGetLastError();
}

}  // namespace sagesla
