// K2: pooled block scores and top-k selection (gfx950).
//
// "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn), §三(二) SLA item 1 keeps the top-k (10%)
// most important regions; "TurboDiffusion技术指南" (blog.gitcode.com) sets that fraction with --sla_topk.
// Importance of key block J for query block I is the dot product of their block means (raw Q, smoothed K);
// the 1/sqrt(D) factor and a softmax over J keep the order, so ranking the dot products selects the same set.
// Exact ties go to the lower J. The output lists are ascending.
//
// Precision: the scores are fp64, so the GPU's ranking can differ from an exact ranking only where two scores
// are within ~1e-13 relative of each other.
#include "device_common.h"
#include "internal.h"

namespace sagesla {

// ---------------------------------------------------------------------------------------------------------
// scores[bh][I][J] = sum_c q_pool[bh][I][c] * k_pool[bh][J][c]   (fp64, fixed order over c)
// grid (ceil(n_kb/128), ceil(n_qb/128), BH), 256 threads; thread (tx, ty) = (t%16, t/16) owns rows
// ty + 16 i and columns tx + 16 j (i, j < 8) of the 128×128 tile. Channels are staged 16 at a time in LDS,
// stored transposed so a wave reads 16 consecutive doubles of the key tile and broadcasts the query tile.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k2_scores(const double* __restrict__ qp, const double* __restrict__ kp,
                                                double* __restrict__ sc, int n_qb, int n_kb) {
  constexpr int TM = 128, TN = 128, KC = 16;
  __shared__ double As[KC][TM];
  __shared__ double Bs[KC][TN];
  const int bh = blockIdx.z;
  const int I0 = blockIdx.y * TM, J0 = blockIdx.x * TN;
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const double* qb = qp + (size_t)bh * n_qb * kD;
  const double* kb = kp + (size_t)bh * n_kb * kD;
  double acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
  const int lr = t >> 1, lc = (t & 1) * 8;  // loader: tile row, first channel of its 8
  for (int c0 = 0; c0 < kD; c0 += KC) {
    double av[8], bv[8];
    const int I = I0 + lr, J = J0 + lr;
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      double2 a = make_double2(0.0, 0.0), b = make_double2(0.0, 0.0);
      if (I < n_qb) a = *(const double2*)(qb + (size_t)I * kD + c0 + lc + u);
      if (J < n_kb) b = *(const double2*)(kb + (size_t)J * kD + c0 + lc + u);
      av[u] = a.x; av[u + 1] = a.y;
      bv[u] = b.x; bv[u + 1] = b.y;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      As[lc + u][lr] = av[u];
      Bs[lc + u][lr] = bv[u];
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < KC; ++c) {
      double a[8], b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = As[c][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = Bs[c][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
  }
  double* out = sc + (size_t)bh * n_qb * n_kb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int I = I0 + ty + 16 * i;
    if (I >= n_qb) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int J = J0 + tx + 16 * j;
      if (J < n_kb) out[(size_t)I * n_kb + J] = acc[i][j] + 0.0;  // +0.0 turns -0 into +0
    }
  }
}

// ---------------------------------------------------------------------------------------------------------
// Top-k per row: one wave per (bh, I) row of scores.
//   flags[J]: 0 dropped, 1 kept, 2 still a candidate.
// Bucket passes: the candidates' value range [lo, hi] is cut into 256 equal bins (the bin of a score is a
// monotone function of it, so bins never reorder scores); the bin holding the k-th best is found from an LDS
// histogram, higher bins are kept, lower ones dropped, and that bin stays candidate. Each pass shrinks the
// range 256-fold, so a few passes leave either <= 256 candidates, ranked exactly by (score desc, J asc), or
// candidates that are all equal, taken in ascending J.
// ---------------------------------------------------------------------------------------------------------
constexpr int kCandMax = 256;
constexpr int kMaxPasses = 16;

__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int l = threadIdx.x & 63;
  return l ? (~0ull >> (64 - l)) : 0ull;
}

__device__ __forceinline__ double wave_min_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmin(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(64) void k2_topk(const double* __restrict__ sc, int32_t* __restrict__ idx, int n_kb,
                                             int topk, int rows) {
  extern __shared__ unsigned char smem[];
  unsigned int* hist = (unsigned int*)smem;                      // 256
  double* cand_s = (double*)(smem + 1024);                       // kCandMax
  int* cand_j = (int*)(smem + 1024 + 8 * kCandMax);              // kCandMax
  unsigned char* flags = smem + 1024 + 12 * kCandMax;            // n_kb
  unsigned char* bins = flags + n_kb;                            // n_kb

  const int row = blockIdx.x;
  if (row >= rows) return;
  const int l = threadIdx.x;
  const double* s = sc + (size_t)row * n_kb;
  int32_t* out = idx + (size_t)row * topk;

  if (topk == 0) return;
  if (topk >= n_kb) {
    for (int J = l; J < n_kb; J += 64) out[J] = J;
    return;
  }

  // initial candidates: everything
  double lo = INFINITY, hi = -INFINITY;
  for (int J = l; J < n_kb; J += 64) {
    flags[J] = 2;
    const double v = s[J];
    lo = fmin(lo, v);
    hi = fmax(hi, v);
  }
  lo = wave_min_f64(lo);
  hi = wave_max_f64(hi);
  int need = topk;       // still to take from the candidates
  int ncand = n_kb;
  bool tie_mode = false;  // candidates all equal: take the lowest J
  __syncthreads();

  for (int pass = 0; pass < kMaxPasses; ++pass) {
    if (need == ncand) {  // every candidate is kept
      for (int J = l; J < n_kb; J += 64)
        if (flags[J] == 2) flags[J] = 1;
      ncand = 0;
      need = 0;
      break;
    }
    if (ncand <= kCandMax) break;
    const double scale = 256.0 / (hi - lo);
    if (!(hi > lo) || !(scale < 1e300)) {
      tie_mode = (hi == lo);
      break;
    }
    for (int b = l; b < 256; b += 64) hist[b] = 0;
    __syncthreads();
    for (int J = l; J < n_kb; J += 64) {
      if (flags[J] != 2) continue;
      int b = (int)((s[J] - lo) * scale);
      b = min(max(b, 0), 255);
      bins[J] = (unsigned char)b;
      atomicAdd(&hist[b], 1u);
    }
    __syncthreads();
    // lane l owns bins 4l..4l+3; find the bin holding the need-th largest candidate
    unsigned int h[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) h[u] = hist[4 * l + u];
    const int mine = (int)(h[0] + h[1] + h[2] + h[3]);
    // count of candidates in bins above lane l's four: inclusive suffix sum over lanes > l
    int suf = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_down(suf, o);
      if (l + o < 64) suf += v;
    }
    int above = suf - mine;  // candidates in bins > 4l+3
    int tbin = -1, tabove = 0, tcnt = 0;
#pragma unroll
    for (int u = 3; u >= 0; --u) {
      const int c = (int)h[u];
      if (tbin < 0 && above < need && need <= above + c) {
        tbin = 4 * l + u;
        tabove = above;
        tcnt = c;
      }
      above += c;
    }
    const unsigned long long found = __ballot(tbin >= 0);
    const int src = __ffsll((long long)found) - 1;
    tbin = __shfl(tbin, src);
    tabove = __shfl(tabove, src);
    tcnt = __shfl(tcnt, src);
    // reclassify and measure the new candidates' range
    lo = INFINITY;
    hi = -INFINITY;
    for (int J = l; J < n_kb; J += 64) {
      if (flags[J] != 2) continue;
      const int b = bins[J];
      if (b > tbin) {
        flags[J] = 1;
      } else if (b < tbin) {
        flags[J] = 0;
      } else {
        const double v = s[J];
        lo = fmin(lo, v);
        hi = fmax(hi, v);
      }
    }
    lo = wave_min_f64(lo);
    hi = wave_max_f64(hi);
    need -= tabove;
    ncand = tcnt;
    __syncthreads();
  }

  if (!tie_mode && ncand > 0 && need > 0 && ncand <= kCandMax) {
    // gather candidates in ascending J, then rank each by (score desc, J asc)
    int base = 0;
    for (int J0 = 0; J0 < n_kb; J0 += 64) {
      const int J = J0 + l;
      const bool c = J < n_kb && flags[J] == 2;
      const unsigned long long m = __ballot(c);
      if (c) {
        const int pos = base + __popcll(m & lanemask_lt());
        cand_s[pos] = s[J];
        cand_j[pos] = J;
      }
      base += __popcll(m);
    }
    __syncthreads();
    for (int i = l; i < ncand; i += 64) {
      const double v = cand_s[i];
      const int J = cand_j[i];
      int rank = 0;
      for (int u = 0; u < ncand; ++u) {
        const double w = cand_s[u];
        rank += (w > v) || (w == v && cand_j[u] < J);
      }
      flags[J] = rank < need ? 1 : 0;
    }
    need = 0;
    __syncthreads();
  } else if (!tie_mode && ncand > kCandMax) {
    tie_mode = true;  // unreachable for finite scores (the range shrinks to one value first); keep lowest J
  }

  // emit kept blocks ascending; in tie mode the first `need` candidates by J are kept as well
  int written = 0, cand_seen = 0;
  for (int J0 = 0; J0 < n_kb; J0 += 64) {
    const int J = J0 + l;
    const int f = J < n_kb ? flags[J] : 0;
    const unsigned long long mc = __ballot(f == 2);
    const int crank = cand_seen + __popcll(mc & lanemask_lt());
    const bool sel = (f == 1) || (tie_mode && f == 2 && crank < need);
    const unsigned long long ms = __ballot(sel);
    if (sel) {
      const int pos = written + __popcll(ms & lanemask_lt());
      if (pos < topk) out[pos] = J;
    }
    written += __popcll(ms);
    cand_seen += __popcll(mc);
  }
}

hipError_t launch_scores(const Plan& p, hipStream_t s) {
  const dim3 grid((p.n_kb + 127) / 128, (p.n_qb + 127) / 128, p.BH);
  hipLaunchKernelGGL(k2_scores, grid, dim3(256), 0, s, p.q_pool, p.k_pool, p.scores, p.n_qb, p.n_kb);
  return hipGetLastError();
}

size_t topk_lds_bytes(int n_kb) { return 1024 + 12 * kCandMax + 2 * (size_t)n_kb; }

hipError_t launch_topk(const Plan& p, hipStream_t s) {
  const int rows = p.BH * p.n_qb;
  hipLaunchKernelGGL(k2_topk, dim3(rows), dim3(64), topk_lds_bytes(p.n_kb), s, p.scores, p.block_idx, p.n_kb,
                     p.topk, rows);
  return hipGetLastError();
}

}  // namespace sagesla
