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
// scores[bh][I][J] = sum_c q_pool[bh][I][c] * k_pool[bh][J][c]   (fp64)
// grid (ceil(n_kb/128), ceil(n_qb/128), BH), 256 threads, fp64 MFMA (v_mfma_f64_16x16x4f64): wave w owns the
// 64x64 quarter (rows 64 (w / 2), columns 64 (w % 2)) of the 128x128 tile as 4x4 accumulator tiles of 16x16.
// Channels are staged 16 at a time in LDS, transposed ([channel][row], rows padded to 136 doubles), and the next
// 16 are loaded into registers during the products of the current ones. Lane layout of the instruction (checked
// on the device): A operand lane l = A[l % 16][l / 16], B operand lane l = B[l / 16][l % 16], accumulator lane l
// element i = D[4 i + l / 16][l % 16]. The products of a step enter the sums in the unit's order, so a score can
// differ from a sequential sum in its last bits; the selection treats scores that close as near-ties.
// ---------------------------------------------------------------------------------------------------------
typedef double v4d __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256, 2) void k2_scores(const double* __restrict__ qp, const double* __restrict__ kp,
                                                   double* __restrict__ sc, int n_qb, int n_kb) {
  constexpr int TM = 128, TN = 128, KC = 16, LD = TM + 8;
  __shared__ double As[KC][LD];
  __shared__ double Bs[KC][LD];
  const int bh = blockIdx.z;
  const int I0 = blockIdx.y * TM, J0 = blockIdx.x * TN;
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  const double* qb = qp + (size_t)bh * n_qb * kD;
  const double* kb = kp + (size_t)bh * n_kb * kD;
  const int lr = t >> 1, lc = (t & 1) * 8;  // loader: tile row, first channel of its 8
  const int I = I0 + lr, J = J0 + lr;
  double av[8], bv[8];
  auto load = [&](int c0) {
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      double2 x = make_double2(0.0, 0.0), y = make_double2(0.0, 0.0);
      if (I < n_qb) x = *(const double2*)(qb + (size_t)I * kD + c0 + lc + u);
      if (J < n_kb) y = *(const double2*)(kb + (size_t)J * kD + c0 + lc + u);
      av[u] = x.x; av[u + 1] = x.y;
      bv[u] = y.x; bv[u + 1] = y.y;
    }
  };
  v4d acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = (v4d){0.0, 0.0, 0.0, 0.0};
  load(0);
  for (int c0 = 0; c0 < kD; c0 += KC) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      As[lc + u][lr] = av[u];
      Bs[lc + u][lr] = bv[u];
    }
    __syncthreads();
    if (c0 + KC < kD) load(c0 + KC);
#pragma unroll
    for (int ks = 0; ks < KC / 4; ++ks) {
      const int kk = 4 * ks + (l >> 4);
      double a[4], b[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) a[mt] = As[kk][wm + 16 * mt + (l & 15)];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) b[nt] = Bs[kk][wn + 16 * nt + (l & 15)];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
    }
  }
  double* out = sc + (size_t)bh * n_qb * n_kb;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int Ir = I0 + wm + 16 * mt + 4 * i + (l >> 4);
      if (Ir >= n_qb) continue;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int Jc = J0 + wn + 16 * nt + (l & 15);
        if (Jc < n_kb) out[(size_t)Ir * n_kb + Jc] = acc[mt][nt][i] + 0.0;  // +0.0 turns -0 into +0
      }
    }
}

// ---------------------------------------------------------------------------------------------------------
// Top-k per row: one wave per (bh, I) row of scores.
//   flags[J]: 0 dropped, 1 kept, 2 still a candidate.
// Histogram passes: every candidate gets a bin 0..255 that is a monotone function of its score (equal scores
// share a bin, a higher score never gets a lower bin); the bin holding the need-th best candidate is found from
// an LDS histogram, higher bins are kept, lower ones dropped, and that bin stays candidate. Value-range passes
// cut the candidates' range [lo, hi] into 256 equal bins, which shrinks it 256-fold per pass on ordinary
// scores; when they stall (scores spread over many binades, or a range beyond fp64) radix passes take the
// candidates' order-preserving 64-bit keys one byte at a time from the top, which ends in at most 8 passes with
// candidates of one key, i.e. one score. Then either <= 256 candidates are ranked exactly by (score desc, J
// asc), or candidates that are all equal are taken in ascending J.
// ---------------------------------------------------------------------------------------------------------
constexpr int kCandMax = 256;
constexpr int kTopkBatch = 8;  // scores per lane loaded together in a pass over the row
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

// unsigned key with the order of the doubles (finite values, -0 == +0 excluded by the score kernel's +0.0):
// negatives have every bit flipped, non-negatives get the sign bit set
__device__ __forceinline__ unsigned long long order_key(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
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

  // initial candidates: everything. The row's loops take the scores kTopkBatch per lane at a time, all loads
  // issued before the first is used, so that each pass waits for memory once per batch rather than per score.
  double lo = INFINITY, hi = -INFINITY;
  for (int J0 = l; J0 < n_kb; J0 += 64 * kTopkBatch) {
    double v[kTopkBatch];
#pragma unroll
    for (int u = 0; u < kTopkBatch; ++u) {
      const int J = J0 + 64 * u;
      v[u] = J < n_kb ? s[J] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < kTopkBatch; ++u) {
      const int J = J0 + 64 * u;
      if (J < n_kb) {
        flags[J] = 2;
        lo = fmin(lo, v[u]);
        hi = fmax(hi, v[u]);
      }
    }
  }
  lo = wave_min_f64(lo);
  hi = wave_max_f64(hi);
  int need = topk;       // still to take from the candidates
  int ncand = n_kb;
  bool tie_mode = false;  // candidates all equal: take the lowest J
  __syncthreads();

  // One histogram pass with the monotone bin function bin_of(score) in [0, 255] over the candidates; afterwards
  // the candidates are those of the bin holding the need-th best, with their score range in [lo, hi].
  auto hist_pass = [&](auto bin_of) {
    for (int b = l; b < 256; b += 64) hist[b] = 0;
    __syncthreads();
    for (int J0 = l; J0 < n_kb; J0 += 64 * kTopkBatch) {
      double v[kTopkBatch];
      bool c[kTopkBatch];
#pragma unroll
      for (int u = 0; u < kTopkBatch; ++u) {
        const int J = J0 + 64 * u;
        c[u] = J < n_kb && flags[J] == 2;
        v[u] = c[u] ? s[J] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < kTopkBatch; ++u) {
        if (!c[u]) continue;
        const int b = bin_of(v[u]);
        bins[J0 + 64 * u] = (unsigned char)b;
        atomicAdd(&hist[b], 1u);
      }
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
    for (int J0 = l; J0 < n_kb; J0 += 64 * kTopkBatch) {
      double v[kTopkBatch];
      bool c[kTopkBatch];
#pragma unroll
      for (int u = 0; u < kTopkBatch; ++u) {
        const int J = J0 + 64 * u;
        int b = -1;
        if (J < n_kb && flags[J] == 2) {
          b = bins[J];
          if (b > tbin)
            flags[J] = 1;
          else if (b < tbin)
            flags[J] = 0;
        }
        c[u] = b == tbin;
        v[u] = c[u] ? s[J] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < kTopkBatch; ++u)
        if (c[u]) {
          lo = fmin(lo, v[u]);
          hi = fmax(hi, v[u]);
        }
    }
    lo = wave_min_f64(lo);
    hi = wave_max_f64(hi);
    need -= tabove;
    ncand = tcnt;
    __syncthreads();
  };
  // when every remaining candidate is to be kept
  auto keep_all = [&]() {
    for (int J = l; J < n_kb; J += 64)
      if (flags[J] == 2) flags[J] = 1;
    ncand = 0;
    need = 0;
    __syncthreads();
  };

  bool done = false;
  for (int pass = 0; pass < kMaxPasses && !done; ++pass) {
    if (need == ncand) {
      keep_all();
      done = true;
    } else if (ncand <= kCandMax) {
      done = true;
    } else if (!(hi > lo)) {
      tie_mode = true;  // every candidate has the same score
      done = true;
    } else {
      const double range = hi - lo;
      if (!(range < INFINITY)) break;  // beyond fp64: the radix passes take over
      // (s - lo) <= range, both rounded monotonically, so the ratio is in [0, 1]
      hist_pass([&](double x) { return min(max((int)((x - lo) / range * 256.0), 0), 255); });
    }
  }
  if (!done) {
    // radix passes over the order-preserving keys, most significant byte first; after the last one the
    // candidates share one key, i.e. one score
    for (int d = 7; d >= 0; --d) {
      if (need == ncand) {
        keep_all();
        break;
      }
      if (ncand <= kCandMax) break;
      hist_pass([&](double x) { return (int)((order_key(x) >> (8 * d)) & 255ull); });
    }
    if (need > 0 && need == ncand)
      keep_all();
    else if (need > 0 && ncand > kCandMax)
      tie_mode = true;  // one key left among the candidates: equal scores
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
