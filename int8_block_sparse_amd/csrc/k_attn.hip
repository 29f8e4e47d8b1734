// K3: block-sparse INT8 flash attention over the selected key blocks (gfx950).
//
// "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn), §三(一) item 3 runs the attention matmuls on
// low-bit matrix units with a restructured softmax; §三(二) item 3 (SageSLA) first selects the important
// regions and runs the INT8 attention only there. For a query block I and each selected key block J:
//   z_ij = (codeQ_i . codeK_j) * scale_q(I) * scale_k(J) * sm_scale      (int32 dot product, exact)
//   O_s[i] = sum_j exp(z_ij - m_i) v_j / sum_j exp(z_ij - m_i)            (online softmax over the selected keys)
// and the epilogue writes out = bf16(O_s + O_lin).
//
// Layout of the work: one workgroup per (b, h, I), BLKQ/32 waves, each wave owns 32 query rows. Scores are
// computed transposed, S^T = K Q^T (v_mfma_i32_32x32x32_i8), so in the accumulator every lane holds one query
// row (lane % 32) and half of the block's 64 keys: row max and row sum are in-lane work plus one exchange
// between the two 32-lane halves. P (bf16) then feeds O^T = V^T P^T (v_mfma_f32_32x32x16_bf16) directly from
// registers; V^T is staged in LDS with its keys ordered to match P's register order. K codes and V^T of the
// next selected block are fetched while the current one is computed (double-buffered LDS).
// Softmax rescaling is lazy: the running max moves only when a block's max exceeds it by more than 2^8, which
// keeps every exp2 argument <= 8 and skips the O rescale for almost every block.
#include "device_common.h"
#include "internal.h"

namespace sagesla {

__device__ __forceinline__ int key_pos16(int off) {  // see V^T layout: slot (g, i) <-> key 8(i/4)+4g+(i%4)
  return (off & 3) | ((off & 4) << 1) | ((off & 8) >> 1);
}

template <int NW>
struct AttnTile {
  static constexpr int NT = NW * 64;
  static constexpr int KU = 512 / NT;  // 16-byte chunks of the 8 KB K tile per thread
  static constexpr int VU = 256 / NT;  // (8 channels x 4 keys) units of the V tile per thread
};

template <int NW>
__device__ __forceinline__ void attn_gload(const int8_t* __restrict__ kb, const uint16_t* __restrict__ vb, int nv,
                                           uint4* rk, uint4* rv) {
  using T = AttnTile<NW>;
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < T::KU; ++u) {
    const int c = t + T::NT * u, r = c >> 3;
    rk[u] = (r < nv) ? *(const uint4*)(kb + r * kD + (c & 7) * 16) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < T::VU; ++u) {
    const int unit = t + T::NT * u, cg = unit & 15, kg = unit >> 4;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = 4 * kg + b;
      rv[4 * u + b] = (r < nv) ? *(const uint4*)(vb + r * kD + cg * 8) : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int NW>
__device__ __forceinline__ void attn_lstore(unsigned char* sk, unsigned char* sv, const uint4* rk, const uint4* rv) {
  using T = AttnTile<NW>;
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < T::KU; ++u) {
    const int c = t + T::NT * u, r = c >> 3, ch = c & 7;
    *(uint4*)(sk + r * 128 + ((ch ^ swz8(r)) << 4)) = rk[u];
  }
#pragma unroll
  for (int u = 0; u < T::VU; ++u) {
    const int unit = t + T::NT * u, cg = unit & 15, kg = unit >> 4;
    const int pos = 16 * (kg >> 2) + key_pos16(4 * (kg & 3));  // 4 consecutive positions for keys 4kg..4kg+3
    const uint32_t w0[4] = {rv[4 * u].x, rv[4 * u].y, rv[4 * u].z, rv[4 * u].w};
    const uint32_t w1[4] = {rv[4 * u + 1].x, rv[4 * u + 1].y, rv[4 * u + 1].z, rv[4 * u + 1].w};
    const uint32_t w2[4] = {rv[4 * u + 2].x, rv[4 * u + 2].y, rv[4 * u + 2].z, rv[4 * u + 2].w};
    const uint32_t w3[4] = {rv[4 * u + 3].x, rv[4 * u + 3].y, rv[4 * u + 3].z, rv[4 * u + 3].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = cg * 8 + e;
      const int sh = (e & 1) * 16;
      const uint32_t k0 = (w0[e >> 1] >> sh) & 0xffffu, k1 = (w1[e >> 1] >> sh) & 0xffffu;
      const uint32_t k2 = (w2[e >> 1] >> sh) & 0xffffu, k3 = (w3[e >> 1] >> sh) & 0xffffu;
      *(uint2*)(sv + row * 128 + (((pos >> 3) ^ swz8(row)) << 4) + ((pos & 7) << 1)) =
          make_uint2(k0 | (k1 << 16), k2 | (k3 << 16));
    }
  }
}

// exp2 of the block's scores, packed to bf16 pairs in PV B-operand order; returns the lane's sum of p.
template <bool RAGGED>
__device__ __forceinline__ float attn_softmax_tile(const v16i& s, float c, float m, int kbase, int nv,
                                                   uint32_t* pw) {
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    float p0 = __builtin_amdgcn_exp2f(fmaf((float)s[r], c, -m));
    float p1 = __builtin_amdgcn_exp2f(fmaf((float)s[r + 1], c, -m));
    if (RAGGED) {
      const int key = kbase + 8 * (r >> 2) + (r & 3);
      p0 = key < nv ? p0 : 0.f;
      p1 = key + 1 < nv ? p1 : 0.f;
    }
    sum += p0 + p1;
    pw[r >> 1] = pack_bf16x2(p0, p1);
  }
  return sum;
}

template <int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void k3_attn(const int8_t* __restrict__ q8, const int8_t* __restrict__ k8,
                                                  const uint16_t* __restrict__ v, const float* __restrict__ qs,
                                                  const float* __restrict__ ks, const int32_t* __restrict__ idx,
                                                  const float* __restrict__ o_lin, uint16_t* __restrict__ out,
                                                  int N, int n_qb, int n_kb, int topk, float c0, int total) {
  constexpr int BLKQ = 32 * NW;
  using T = AttnTile<NW>;
  __shared__ __attribute__((aligned(16))) unsigned char s_k[2][64 * 128];
  __shared__ __attribute__((aligned(16))) unsigned char s_v[2][128 * 128];

  const int item = xcd_remap(blockIdx.x, total);
  const int bh = item / n_qb, I = item % n_qb;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 5, lr = l & 31;
  const int row = I * BLKQ + 32 * w + lr;
  const bool rok = row < N;

  v4i bq[4];
  {
    const int8_t* qrow = q8 + ((size_t)bh * N + (rok ? row : 0)) * kD;
#pragma unroll
    for (int s = 0; s < 4; ++s) bq[s] = rok ? *(const v4i*)(qrow + 32 * s + 16 * g) : (v4i){0, 0, 0, 0};
  }
  const float cq = qs[(size_t)bh * n_qb + I] * c0;
  const int32_t* irow = idx + ((size_t)bh * n_qb + I) * topk;
  const int8_t* kbase = k8 + (size_t)bh * N * kD;
  const uint16_t* vbase = v + (size_t)bh * N * kD;
  const float* ksrow = ks + (size_t)bh * n_kb;

  v16f o[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) o[ct] = (v16f){};
  float m_run = -INFINITY, l_run = 0.f;

  uint4 rk[T::KU], rv[4 * T::VU];
  if (topk > 0) {
    {
      const int J = min(max(irow[0], 0), n_kb - 1);
      attn_gload<NW>(kbase + (size_t)J * kBlkK * kD, vbase + (size_t)J * kBlkK * kD, min(kBlkK, N - J * kBlkK), rk, rv);
      attn_lstore<NW>(s_k[0], s_v[0], rk, rv);
    }
    __syncthreads();
    for (int j = 0; j < topk; ++j) {
      const int buf = j & 1;
      if (j + 1 < topk) {
        const int Jn = min(max(irow[j + 1], 0), n_kb - 1);
        attn_gload<NW>(kbase + (size_t)Jn * kBlkK * kD, vbase + (size_t)Jn * kBlkK * kD,
                       min(kBlkK, N - Jn * kBlkK), rk, rv);
      }
      const int J = min(max(irow[j], 0), n_kb - 1);
      const int nv = min(kBlkK, N - J * kBlkK);
      const float c = cq * ksrow[J];
      const unsigned char* sk = s_k[buf];
      const unsigned char* sv = s_v[buf];

      // S^T = K Q^T for keys 0..31 (tile 0) and 32..63 (tile 1)
      v16i sacc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        sacc[tt] = (v16i){};
        const int kr = 32 * tt + lr;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const v4i a = *(const v4i*)(sk + kr * 128 + (((2 * s + g) ^ swz8(kr)) << 4));
          sacc[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq[s], sacc[tt], 0, 0, 0);
        }
      }
      // lane (row lr, half g) holds key 32tt + 8(r/4) + 4g + (r%4) in sacc[tt][r]
      const bool ragged = nv < kBlkK;
      int mx = INT_MIN;
      if (!ragged) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = max(mx, sacc[tt][r]);
      } else {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * tt + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key < nv) mx = max(mx, sacc[tt][r]);
          }
      }
      mx = max(mx, swap_halves_i32(mx));
      const float mblk = (float)mx * c;
      const bool need = mblk > m_run + 8.f;
      if (__ballot(need)) {
        const float m_new = need ? mblk : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
        m_run = m_new;
      }
      uint32_t pw[2][8];
      float ps;
      if (!ragged) {
        ps = attn_softmax_tile<false>(sacc[0], c, m_run, 4 * g, nv, pw[0]) +
             attn_softmax_tile<false>(sacc[1], c, m_run, 32 + 4 * g, nv, pw[1]);
      } else {
        ps = attn_softmax_tile<true>(sacc[0], c, m_run, 4 * g, nv, pw[0]) +
             attn_softmax_tile<true>(sacc[1], c, m_run, 32 + 4 * g, nv, pw[1]);
      }
      l_run += ps;

      // O^T += V^T P^T: step s covers keys 16s..16s+15 = registers 8(s%2)..+7 of tile s/2
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t* p = pw[s >> 1] + 4 * (s & 1);
        const v8bf b = __builtin_bit_cast(v8bf, make_uint4(p[0], p[1], p[2], p[3]));
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int vr = 32 * ct + lr;
          const v8bf a = *(const v8bf*)(sv + vr * 128 + (((2 * s + g) ^ swz8(vr)) << 4));
          o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[ct], 0, 0, 0);
        }
      }
      if (j + 1 < topk) attn_lstore<NW>(s_k[buf ^ 1], s_v[buf ^ 1], rk, rv);
      __syncthreads();
    }
  }

  const float lt = l_run + swap_halves_f32(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (rok) {
    const size_t ro = ((size_t)bh * N + row) * kD;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int e0 = 32 * ct + 8 * r4 + 4 * g;
        float x0 = o[ct][4 * r4] * inv, x1 = o[ct][4 * r4 + 1] * inv;
        float x2 = o[ct][4 * r4 + 2] * inv, x3 = o[ct][4 * r4 + 3] * inv;
        if (o_lin) {
          const float4 a = *(const float4*)(o_lin + ro + e0);
          x0 += a.x; x1 += a.y; x2 += a.z; x3 += a.w;
        }
        *(uint2*)(out + ro + e0) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
      }
  }
}

hipError_t launch_attn(const Plan& p, const uint16_t* v, uint16_t* out, hipStream_t s) {
  const int total = p.BH * p.n_qb;
  const float c0 = p.sm_scale * 1.4426950408889634f;  // log2(e): scores enter exp2
  const float* olin = (p.linear && p.topk < p.n_kb) ? p.o_lin : nullptr;
  if (p.blk_q == 128)
    hipLaunchKernelGGL(k3_attn<4>, dim3(total), dim3(256), 0, s, p.q_i8, p.k_i8, v, p.q_scale, p.k_scale,
                       p.block_idx, olin, out, p.N, p.n_qb, p.n_kb, p.topk, c0, total);
  else
    hipLaunchKernelGGL(k3_attn<2>, dim3(total), dim3(128), 0, s, p.q_i8, p.k_i8, v, p.q_scale, p.k_scale,
                       p.block_idx, olin, out, p.N, p.n_qb, p.n_kb, p.topk, c0, total);
  return hipGetLastError();
}

}  // namespace sagesla
