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
// registers; V^T is staged in LDS with its keys ordered to match P's register order (the quantize kernel writes
// each key block's V^T once as a ready LDS image). K codes and the V^T image of the next selected block are
// loaded straight into the idle LDS buffer (global_load_lds) while the current one is computed.
// Softmax rescaling is lazy: the running max moves only when a block's max exceeds it by more than 2^8, which
// keeps every exp2 argument <= 8 and skips the O rescale for almost every block.
#include "device_common.h"
#include "internal.h"

namespace sagesla {

template <int NW>
struct AttnTile {
  static constexpr int NT = NW * 64;
  static constexpr int KPW = 8 / NW;   // 1 KB (64 lanes x 16 B) direct-to-LDS loads per wave for the 8 KB K tile
  static constexpr int VPW = 16 / NW;  // ... and for the 16 KB V^T image
};

typedef __attribute__((address_space(3))) void lds_void;

// Stage key block J into one LDS buffer with direct global->LDS loads (no registers, no VALU work):
// the K codes land row-major with 16-byte chunks XOR-swizzled per row, the V^T image is copied verbatim
// (it was written in its LDS layout by the quantize kernel). Rows past the end of a ragged block re-read the
// last valid row; their scores are masked and their V^T columns are zero.
template <int NW>
__device__ __forceinline__ void attn_stage(const int8_t* __restrict__ kb, const unsigned char* __restrict__ vimg,
                                           int nv, unsigned char* sk, unsigned char* sv) {
  using T = AttnTile<NW>;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < T::KPW; ++i) {
    const int blk = w * T::KPW + i;
    const int p = blk * 64 + l;  // 16-byte position in the LDS image
    const int r = p >> 3, ch = (p & 7) ^ swz8(r);
    const int8_t* src = kb + min(r, nv - 1) * kD + ch * 16;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(sk + blk * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < T::VPW; ++i) {
    const int blk = w * T::VPW + i;
    __builtin_amdgcn_global_load_lds((const void*)(vimg + (blk * 64 + l) * 16), (lds_void*)(sv + blk * 1024), 16, 0,
                                     0);
  }
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One selected key block: S^T on INT8 MFMA, online softmax update, O^T += V^T P^T on BF16 MFMA.
// Lane (row lr, half g) holds key 32tt + 8(r/4) + 4g + (r%4) of the block in s[tt][r].
template <bool RAGGED>
__device__ __forceinline__ void attn_block(const unsigned char* sk, const unsigned char* sv, const v4i* bq,
                                           const int (&koff)[2][4], const int (&voff)[4][4], float c, int nv,
                                           int g, v16f* o, float& m_run, float& l_run) {
  v16i sacc[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    sacc[tt] = (v16i){};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v4i a = *(const v4i*)(sk + koff[tt][s]);
      sacc[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq[s], sacc[tt], 0, 0, 0);
    }
  }
  int mx = INT_MIN;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (RAGGED) {
        const int key = 32 * tt + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= nv) sacc[tt][r] = INT_MIN;
      }
      mx = max(mx, sacc[tt][r]);
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
  // p = exp2(s*c - m), packed to bf16 pairs in the order of the PV B operand; the row sum is taken over the
  // same bf16 values the PV product uses
  uint32_t pw[2][8];
  float ps = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0 = __builtin_amdgcn_exp2f(fmaf((float)sacc[tt][r], c, -m_run));
      float p1 = __builtin_amdgcn_exp2f(fmaf((float)sacc[tt][r + 1], c, -m_run));
      if (RAGGED) {
        p0 = sacc[tt][r] == INT_MIN ? 0.f : p0;
        p1 = sacc[tt][r + 1] == INT_MIN ? 0.f : p1;
      }
      const uint32_t pk = pack_bf16x2(p0, p1);
      pw[tt][r >> 1] = pk;
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, pk), (v2bf){(__bf16)1.0f, (__bf16)1.0f}, ps,
                                           false);
    }
  l_run += ps;
  // O^T += V^T P^T: step s covers keys 16s..16s+15 = registers 8(s%2)..+7 of tile s/2
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t* p = pw[s >> 1] + 4 * (s & 1);
    const v8bf b = __builtin_bit_cast(v8bf, make_uint4(p[0], p[1], p[2], p[3]));
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const v8bf a = *(const v8bf*)(sv + voff[ct][s]);
      o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[ct], 0, 0, 0);
    }
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void k3_attn(
    const int8_t* __restrict__ q8, const int8_t* __restrict__ k8, const unsigned char* __restrict__ vt,
    const float* __restrict__ qs, const float* __restrict__ ks, const int32_t* __restrict__ idx,
    const float* __restrict__ o_lin, uint16_t* __restrict__ out, int N, int n_qb, int n_kb, int topk, float c0,
    int total) {
  constexpr int BLKQ = 32 * NW;
  __shared__ __attribute__((aligned(1024))) unsigned char s_k[2][64 * 128];
  __shared__ __attribute__((aligned(1024))) unsigned char s_v[2][128 * 128];

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
  // per-lane LDS byte offsets of the MFMA operands inside one buffer
  int koff[2][4], voff[4][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kr = 32 * tt + lr;
      koff[tt][s] = kr * 128 + (((2 * s + g) ^ swz8(kr)) << 4);
    }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int vr = 32 * ct + lr;
      voff[ct][s] = vr * 128 + (((2 * s + g) ^ swz8(vr)) << 4);
    }
  const float cq = qs[(size_t)bh * n_qb + I] * c0;
  const int32_t* irow = idx + ((size_t)bh * n_qb + I) * topk;
  const int8_t* kbase = k8 + (size_t)bh * N * kD;
  const unsigned char* vbase = vt + (size_t)bh * n_kb * 16384;
  const float* ksrow = ks + (size_t)bh * n_kb;

  v16f o[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) o[ct] = (v16f){};
  float m_run = -INFINITY, l_run = 0.f;

  auto stage = [&](int j, int buf) {
    const int J = min(max(irow[j], 0), n_kb - 1);
    attn_stage<NW>(kbase + (size_t)J * kBlkK * kD, vbase + (size_t)J * 16384, min(kBlkK, N - J * kBlkK), s_k[buf],
                   s_v[buf]);
  };
  auto finish = [&]() {
    wait_vmem_all();
    __syncthreads();
  };
  if (topk > 0) {
    // Only the last key block can be ragged. Ascending lists hold it last, so the main loop runs the full-block
    // body only and the ragged block (if selected) is peeled; a caller-given list that places it elsewhere
    // takes the generic loop.
    const int last_kb = n_kb - 1;
    const bool has_ragged = (N % kBlkK) != 0;
    bool tail_ragged = false, elsewhere = false;
    if (has_ragged) {
      tail_ragged = min(max(irow[topk - 1], 0), last_kb) == last_kb;
      for (int j = 0; j < topk - 1; ++j) elsewhere |= min(max(irow[j], 0), last_kb) == last_kb;
    }
    stage(0, 0);
    finish();
    if (!elsewhere) {
      const int nfull = topk - (tail_ragged ? 1 : 0);
      int j = 0;
      for (; j + 1 < nfull; j += 2) {
        stage(j + 1, 1);
        attn_block<false>(s_k[0], s_v[0], bq, koff, voff, cq * ksrow[min(max(irow[j], 0), last_kb)], kBlkK, g, o,
                          m_run, l_run);
        finish();
        if (j + 2 < topk) stage(j + 2, 0);
        attn_block<false>(s_k[1], s_v[1], bq, koff, voff, cq * ksrow[min(max(irow[j + 1], 0), last_kb)], kBlkK, g,
                          o, m_run, l_run);
        finish();
      }
      if (j < nfull) {  // odd count of full blocks: buffer 0 holds block j
        if (j + 1 < topk) stage(j + 1, 1);
        attn_block<false>(s_k[0], s_v[0], bq, koff, voff, cq * ksrow[min(max(irow[j], 0), last_kb)], kBlkK, g, o,
                          m_run, l_run);
        finish();
        ++j;
      }
      if (tail_ragged) {
        const int buf = j & 1;
        attn_block<true>(s_k[buf], s_v[buf], bq, koff, voff, cq * ksrow[last_kb], N - last_kb * kBlkK, g, o,
                         m_run, l_run);
      }
    } else {
      for (int j = 0; j < topk; ++j) {
        const int buf = j & 1;
        if (j + 1 < topk) stage(j + 1, buf ^ 1);
        const int J = min(max(irow[j], 0), last_kb);
        attn_block<true>(s_k[buf], s_v[buf], bq, koff, voff, cq * ksrow[J], min(kBlkK, N - J * kBlkK), g, o, m_run,
                         l_run);
        finish();
      }
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

hipError_t launch_attn(const Plan& p, uint16_t* out, hipStream_t s) {
  const int total = p.BH * p.n_qb;
  const float c0 = p.sm_scale * 1.4426950408889634f;  // log2(e): scores enter exp2
  const float* olin = (p.linear && p.topk < p.n_kb) ? p.o_lin : nullptr;
  if (p.blk_q == 128)
    hipLaunchKernelGGL(k3_attn<4>, dim3(total), dim3(256), 0, s, p.q_i8, p.k_i8, p.v_img, p.q_scale, p.k_scale,
                       p.block_idx, olin, out, p.N, p.n_qb, p.n_kb, p.topk, c0, total);
  else
    hipLaunchKernelGGL(k3_attn<2>, dim3(total), dim3(128), 0, s, p.q_i8, p.k_i8, p.v_img, p.q_scale, p.k_scale,
                       p.block_idx, olin, out, p.N, p.n_qb, p.n_kb, p.topk, c0, total);
  return hipGetLastError();
}

}  // namespace sagesla
