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
// each key block's V^T once as a ready LDS image). K codes and V^T images move through two three-slot LDS rings
// with direct global->LDS loads (global_load_lds) issued two iterations ahead, and each barrier waits only for
// the loads of two iterations back; each iteration computes the next block's scores while it runs this block's
// softmax, and the scheduler interleaves those MFMAs (and the PV MFMAs) with the softmax VALU work so the matrix
// core and the vector ALU of a wave overlap.
// Softmax rescaling is lazy: the running max moves only when a block's max exceeds it by more than kLazy (log2
// units), which keeps every exp2 argument <= kLazy and skips the O rescale for almost every block.
// Bounded shift: the exponent of a softmax may subtract any per-row constant instead of the row max. Each wave
// bounds its rows' scores from above by Cauchy-Schwarz, t_ij <= B_i = |codeQ_i| * scale_q * sm_scale * log2(e) *
// max over the listed J of scale_k(J) * (largest |codeK_j| under that scale, from the quantizer), and when
// B_i - M_i <= kBoundGap for every row, with M_i the row's score against the first key of its first listed block
// (a lower bound of its max), it subtracts m_i = B_i - kBoundTop throughout: every p <= 2^kBoundTop, the row's
// largest p >= 2^(kBoundTop - kBoundGap), so no per-block max, no rescale and no overflow or underflow of the sums.
// Otherwise the wave keeps the lazy running max.
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "lin_common.h"

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
// (it was written in its LDS layout by the quantize kernel). Each lane's source offsets inside a block are
// fixed (koffs for K, (blk*64 + l)*16 for V), so a load is a uniform block base plus a lane offset.
template <int NW>
struct StageOffsets {
  uint32_t k[AttnTile<NW>::KPW];
};

template <int NW>
__device__ __forceinline__ StageOffsets<NW> stage_offsets(int nv) {
  using T = AttnTile<NW>;
  StageOffsets<NW> so;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < T::KPW; ++i) {
    const int p = (w * T::KPW + i) * 64 + l;  // 16-byte position in the LDS image
    const int r = p >> 3, ch = (p & 7) ^ swz32(r);
    so.k[i] = (uint32_t)(min(r, nv - 1) * kD + ch * 16);  // rows past a ragged end re-read the last valid row
  }
  return so;
}

// Buffer descriptor over one (b, h) slab: raw addressing (stride 0), gfx9 descriptor word 3. The tile loads
// are buffer loads to LDS: a uniform block offset in an SGPR plus a per-lane offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// (TAG only gives each attention-kernel instantiation its own specialization: when two kernels with the same NW
// share one, the host compilation pass rejects the call inside the second kernel's lambdas)
template <int NW, int TAG = 0>
__device__ __forceinline__ void stage_k(__amdgpu_buffer_rsrc_t rk, uint32_t blk_off, const StageOffsets<NW>& so,
                                        unsigned char* sk) {
  using T = AttnTile<NW>;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: LDS bases stay scalar
#pragma unroll
  for (int i = 0; i < T::KPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(sk + (w * T::KPW + i) * 1024), 16, so.k[i], blk_off, 0,
                                             0);
}

template <int NW>
__device__ __forceinline__ void stage_v(__amdgpu_buffer_rsrc_t rv, uint32_t blk_off, unsigned char* sv) {
  using T = AttnTile<NW>;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lane_off = (threadIdx.x & 63) * 16;
#pragma unroll
  for (int i = 0; i < T::VPW; ++i) {
    const int blk = w * T::VPW + i;  // 1 KB piece of the image: uniform part in the scalar offset
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(sv + blk * 1024), 16, lane_off, blk_off + blk * 1024, 0,
                                             0);
  }
}

template <int NW, int TAG = 0>
__device__ __forceinline__ void attn_stage(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int J,
                                           const StageOffsets<NW>& so, unsigned char* sk, unsigned char* sv) {
  stage_k<NW, TAG>(rk, (uint32_t)J * (kBlkK * kD), so, sk);
  stage_v<NW>(rv, (uint32_t)J * 16384u, sv);
}

// Wait until at most N of this wave's vector-memory loads are still in flight and its LDS reads have returned,
// then meet the other waves of the workgroup. The direct-to-LDS loads of a wave complete in issue order, so the
// tiles issued before the last N loads have landed in every wave's share once all waves pass the barrier. The
// empty asm statements keep the compiler from moving LDS accesses across the barrier.
// The wait goes through the builtin (s_waitcnt simm16: vmcnt in bits 3:0 and 15:14, expcnt 6:4 left at its
// maximum, lgkmcnt 11:8 = 0) so that the compiler's own counter tracking knows which loads have completed.
template <int N>
__device__ __forceinline__ void ring_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt has six bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Scores of one key block (S^T = K Q^T, 8 INT8 MFMAs into two 32-key tiles). The int32 accumulators start at
// kMagic is the fp32 bit pattern of 1/(2*pi), 0x3E22F983, whose mantissa field 0x22F983 = 2292099 leaves
// 2292099 steps below it and 2^23 - 2292099 = 6096509 above it inside its binade. Since |S| <= 127*127*128 =
// 2064512, the sum read as a float is exactly 2^-3 + (2292099 + S) * 2^-26 (no int-to-float conversion), and since
// the pattern is an inline constant of the instruction set, the first MFMA of each tile takes it as its
// accumulator operand without any register being set up.
constexpr int kMagic = 0x3E22F983;
constexpr int kMagicMant = kMagic & 0x7FFFFF;
constexpr float kMagicF = __builtin_bit_cast(float, kMagic);  // 2^-3 * (1 + kMagicMant * 2^-23)
constexpr float kMagicScale = 0x1p26f;                        // one unit of S in that float is 2^-26
constexpr float kMagicUnits = kMagicF * kMagicScale;          // 2^23 + kMagicMant, exact
static_assert(kMagicUnits == float((1 << 23) + kMagicMant), "the magic's float value in units of S");
static_assert(127 * 127 * 128 < kMagicMant && 127 * 127 * 128 < (1 << 23) - kMagicMant,
              "scores must stay in the binade");
constexpr int kListCap = 1020;  // selection-list entries the attention kernel keeps in LDS
// Lazy-rescale slack in log2 units: probabilities stay <= 2^24, so a row sum over the largest key count stays
// below 2^45, far inside fp32; on smooth video-like inputs a running max of 32 rows moves for under 1% of
// blocks (about 6% with a slack of 8).
constexpr float kLazy = 24.f;
// Bounded shift (see the header): p <= 2^kBoundTop keeps the row sums below 2^(kBoundTop + 17) for any list of
// up to 2^17 keys and O far inside fp32; the largest p of a row is >= 2^(kBoundTop - kBoundGap) = 2^-96, a normal
// fp32 and bf16 value, so the terms that do underflow are below 2^-30 of it.
constexpr float kBoundTop = 64.f;
constexpr float kBoundGap = 160.f;

__device__ __forceinline__ void attn_scores(const unsigned char* __restrict__ sk, const v4i* bq, const int (&koff)[2][4],
                                            v16i (&sacc)[2]) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[tt][r] = kMagic;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v4i a = *(const v4i*)(sk + koff[tt][s]);
      sacc[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq[s], sacc[tt], 0, 0, 0);
    }
  }
}

// One pair of probabilities: p = exp2(S*c - m) for scores r, r+1 of a 32-key tile, packed to bf16 in PV
// B-operand order; the row sum is taken over the same bf16 values the PV product uses. s holds kMagic + S, read as
// the float x = kMagicF + S * 2^-26, and c26 = c * 2^26. FAST: t = fma(x, c26, -kc) = (kMagicUnits + S) * c - kc
// with kc = fl(kMagicUnits * c + m), one instruction; kc's rounding shifts every t of the block by the same
// amount, at most half an ulp of kc (<= 2^-11 for c < 2^-10). Otherwise t = fma(x - kMagicF, c26, -m), where the
// subtraction is exact and the product is S * c: the same value as fma(S, c, -m). Ragged keys carry INT_MIN and
// get p = 0.
template <bool RAGGED, bool FAST>
__device__ __forceinline__ void attn_exp_pair(const v16i& s, int r, float c26, float m, float kc, uint32_t& pk,
                                              float& ps) {
  const float x0 = __int_as_float(s[r]), x1 = __int_as_float(s[r + 1]);
  float p0 = __builtin_amdgcn_exp2f(FAST ? fmaf(x0, c26, -kc) : fmaf(x0 - kMagicF, c26, -m));
  float p1 = __builtin_amdgcn_exp2f(FAST ? fmaf(x1, c26, -kc) : fmaf(x1 - kMagicF, c26, -m));
  if (RAGGED) {
    p0 = s[r] == INT_MIN ? 0.f : p0;
    p1 = s[r + 1] == INT_MIN ? 0.f : p1;
  }
  pk = pack_bf16x2(p0, p1);
  ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, pk), (v2bf){(__bf16)1.0f, (__bf16)1.0f}, ps, false);
}

// One selected key block j whose scores are in scur. With HAS_NEXT the scores of block j+1 (K codes in sk_next)
// are computed into snext in the same pass. Lane (row lr, half g) holds key 32tt + 8(r/4) + 4g + (r%4) of the
// block in scur[tt][r].
//
// The pass is written as a fixed sequence of slots, one MFMA each: first the 8 score MFMAs of the next block
// (S^T tiles tt = 0, 1, steps s = 0..3), then the 16 PV MFMAs of this block (steps s = 0..3, tiles ct = 0..3).
// Each slot also issues the LDS operand read of the MFMA four slots later and one pair of this block's exps,
// which run four pairs ahead of the PV steps that consume them. Scheduling barriers between the slots keep the
// compiler from collapsing the read-ahead distance.
// G (one scale per 32 keys): score tile 0 (keys 0-31) takes the scale product c and tile 1 (keys 32-63) c1;
// otherwise both take c.
template <bool RAGGED, bool HAS_NEXT, bool FAST, bool G = false, bool BOUNDED = false>
__device__ __forceinline__ void attn_iter(const unsigned char* __restrict__ sk_next,
                                          const unsigned char* __restrict__ sv, const v4i* bq,
                                          const int (&koff)[2][4], const int (&voff)[4][4], float c, float c1, int nv,
                                          int g, v16f* o, float& m_run, float& l_run, v16i (&scur)[2],
                                          v16i (&snext)[2]) {
  constexpr int NK = HAS_NEXT ? 8 : 0;  // score MFMAs of the next block
  constexpr int NS = NK + 16;           // MFMAs of the pass
  constexpr int AHEAD = 4;              // operand reads run this many MFMAs ahead
  v4i ka[8];
  v8bf va[16];
  uint32_t pw[16];
  auto read = [&](int i) {
    if (i < NK) {
      ka[i] = *(const v4i*)(sk_next + koff[i >> 2][i & 3]);
    } else {
      const int v = i - NK;
      va[v] = *(const v8bf*)(sv + voff[v & 3][v >> 2]);
    }
  };
  auto mfma = [&](int i) {
    if (i < NK) {
      const int tt = i >> 2, st = i & 3;
      if (st == 0)
        snext[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
            ka[i], bq[st],
            (v16i){kMagic, kMagic, kMagic, kMagic, kMagic, kMagic, kMagic, kMagic, kMagic, kMagic, kMagic, kMagic,
                   kMagic, kMagic, kMagic, kMagic},
            0, 0, 0);
      else
        snext[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[i], bq[st], snext[tt], 0, 0, 0);
    } else {
      const int v = i - NK, st = v >> 2, ct = v & 3;
      const v8bf b = __builtin_bit_cast(v8bf, make_uint4(pw[4 * st], pw[4 * st + 1], pw[4 * st + 2], pw[4 * st + 3]));
      o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[v], b, o[ct], 0, 0, 0);
    }
  };
  // block max over 8 registers of one tile half, ragged keys masked to INT_MIN
  auto part_max = [&](int q) {
    const int tt = q >> 1;
    int mq = INT_MIN;
#pragma unroll
    for (int r = 8 * (q & 1); r < 8 * (q & 1) + 8; ++r) {
      if (RAGGED) {
        const int key = 32 * tt + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= nv) scur[tt][r] = INT_MIN;
      }
      mq = max(mq, scur[tt][r]);
    }
    return mq;
  };

  // region 1: first operand reads; with a next block, its first four score MFMAs overlap the block max
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) read(i);
  // (BOUNDED: m_run is the row's fixed shift; only a ragged block's keys past N are masked)
  int mx = INT_MIN, mx1 = INT_MIN;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (HAS_NEXT) {
      __builtin_amdgcn_sched_barrier(0);
      read(q + AHEAD);
      mfma(q);
    }
    if (!BOUNDED || RAGGED) {
      if (G && q >= 2)
        mx1 = max(mx1, part_max(q));
      else
        mx = max(mx, part_max(q));
    }
  }
  if constexpr (!BOUNDED) {
  mx = max_halves_i32(mx);
  float mblk = (float)(mx - kMagic) * c;
  if constexpr (G) {
    // tile 1 of a ragged block may hold no valid key at all (its max then stays INT_MIN)
    mx1 = max_halves_i32(mx1);
    mblk = fmaxf(mblk, (RAGGED && mx1 == INT_MIN) ? -INFINITY : (float)(mx1 - kMagic) * c1);
  }
  const bool need = mblk > m_run + kLazy;
  if (__ballot(need)) {
    // rare: keep it a real branch (the marker has side effects, so the body is never executed speculatively)
    asm volatile("; rescale running max" ::: "memory");
    const float m_new = need ? mblk : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
    m_run = m_new;
  }
  }

  // region 2: slot k runs MFMA k, the read for MFMA k + AHEAD and exp pair k - NK + 4
  const float kc = FAST ? fmaf(kMagicUnits, c, m_run) : 0.f;
  const float c26 = c * kMagicScale;
  const float kc1 = G ? (FAST ? fmaf(kMagicUnits, c1, m_run) : 0.f) : kc;
  const float c26_1 = G ? c1 * kMagicScale : c26;
  float ps = 0.f;
#pragma unroll
  for (int k = HAS_NEXT ? 4 : -4; k < NS; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    if (k >= 0 && k + AHEAD < NS && k + AHEAD >= (HAS_NEXT ? 8 : AHEAD)) read(k + AHEAD);
    if (k >= 0) mfma(k);
    const int e = k - NK + 4;
    if (e >= 0 && e < 16)
      attn_exp_pair<RAGGED, FAST>(scur[e >> 3], 2 * (e & 7), (e >> 3) ? c26_1 : c26, m_run, (e >> 3) ? kc1 : kc,
                                  pw[e], ps);
  }
  __builtin_amdgcn_sched_barrier(0);
  l_run += ps;
}

// Linear branch of one query block, run at the end of the attention kernel (the ring's LDS is free then):
//   U^T[e][i] = f_e sum_c P^T[e][c] phi'(Q)^T[c][i]   (A = the record's fp16 plane from LDS, B = phi' in registers)
//   O^T[f][i] = sum_e W_p^T[f][e] U^T[e][i]          (A = W_p^T from LDS, B = U^T hi/lo from the accumulators)
// and den[i] = phi'(q_i) . Z_m. The remaining state is H_m^T as an fp16 plane P (rows e, each row 256 B at its own
// place in the head's row-major planes) with one factor f_e per row, and Z_m in fp32 (the aux record), H_m and Z_m
// sharing one power-of-two scale; phi' = phi scaled per row by the power of two that puts the row's largest value
// in [1, 2) (phi is increasing, so that is phi of the row's largest q). Both common factors cancel in U / den.
// Buffer loads gather the plane rows into the ring's V slots (rows 0-63 in v0, 64-127 in v1) and the row factors
// into k2 + 1024, while Z arrives in k2 by ordinary loads and phi' is formed; then W_p^T takes the V slots the same
// way. Wave w handles its own 32 rows. acc2 returns O^T unnormalized in the attention
// accumulators' layout (row lr, channel 32 ft + 8 (r / 4) + 4 g + r % 4) and inv_l = 1 / den.
template <int NW>
__device__ __forceinline__ void lin_epilogue(const uint16_t* __restrict__ q, const unsigned char* __restrict__ plane16,
                                             const unsigned char* __restrict__ aux16,
                                             const uint16_t* __restrict__ wpt, int bh, int I, int N, int n_qb,
                                             unsigned char* __restrict__ k2, unsigned char* __restrict__ v0,
                                             unsigned char* __restrict__ v1, v16f (&acc2)[4], float& inv_l) {
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, g = l >> 5, lr = l & 31;
  constexpr int BLKQ = 32 * NW;
  const unsigned char* sax = aux16 + ((size_t)bh * n_qb + I) * (size_t)kAuxBytes;
  float* s_z = (float*)k2;
  const float* s_f = (const float*)(k2 + 1024);
  __syncthreads();  // every wave is done with the ring slots
  float4 zv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (t < kD / 4) zv = *(const float4*)(sax + kAuxZ + 16 * t);  // issued before the plane loads: waited alone
  {  // the plane: 32 loads of 1 KB, each four rows of 256 B (lane l: row 4k + l / 16, chunk l % 16); the row
     // factors: one load of 1 KB (its second half past the aux record reads 0). Offsets are per lane, so the
     // range check sees all of them.
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(plane16 + (size_t)bh * kD * n_qb * 256), (short)0, kD * n_qb * 256, 0x00020000);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(sax), (short)0, kAuxBytes, 0x00020000);
    const uint32_t lrow = (uint32_t)(((l >> 4) * n_qb + I) * 256 + (l & 15) * 16);
    for (int k = w; k < 33; k += NW) {
      unsigned char* dst = k < 16 ? v0 + k * 1024 : k < 32 ? v1 + (k - 16) * 1024 : k2 + 1024;
      if (k < 32)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (__attribute__((address_space(3))) void*)dst, 16,
                                                 lrow + (uint32_t)(4 * k * n_qb * 256), 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)dst, 16,
                                                 l * 16 + kAuxF, 0, 0, 0);
    }
  }
  if (t < kD / 4) *(float4*)(s_z + 4 * t) = zv;

  const int row = I * BLKQ + 32 * w + lr;
  const bool rok = row < N;
  const uint16_t* qrow = q + ((size_t)bh * N + (rok ? row : 0)) * kD;
  // first pass over the row: its largest q (the row is read again below, from the cache, to keep registers free)
  float qm = -INFINITY;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    uint4 wq = make_uint4(0, 0, 0, 0);
    if (rok) wq = *(const uint4*)(qrow + 16 * s + 8 * g);
    const uint32_t ww[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) qm = fmaxf(qm, fmaxf(bf16_lo(ww[u]), bf16_hi(ww[u])));
  }
  qm = fmaxf(qm, swap_halves_f32(qm));
  int kx = 0;
  (void)frexpf(phi_f(qm), &kx);  // the row's largest phi < 2^kx
  const int sh = 1 - kx;
  const float sc = ldexpf(1.f, sh), shf = (float)sh;
  __syncthreads();  // s_z
  v8h bq16[8];
  float den = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c0 = 16 * s + 8 * g;
    uint4 wq = make_uint4(0, 0, 0, 0);
    if (rok) wq = *(const uint4*)(qrow + c0);
    const uint32_t ww[4] = {wq.x, wq.y, wq.z, wq.w};
    uint32_t hw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x0 = bf16_lo(ww[u]), x1 = bf16_hi(ww[u]);
      const float p0 = x0 > 0.f ? fmaf(x0, sc, sc) : __builtin_amdgcn_exp2f(fmaf(x0, 1.4426950408889634f, shf));
      const float p1 = x1 > 0.f ? fmaf(x1, sc, sc) : __builtin_amdgcn_exp2f(fmaf(x1, 1.4426950408889634f, shf));
      den = fmaf(p0, s_z[c0 + 2 * u], den);
      den = fmaf(p1, s_z[c0 + 2 * u + 1], den);
      hw[u] = pack_f16x2(p0, p1);
    }
    bq16[s] = __builtin_bit_cast(v8h, make_uint4(hw[0], hw[1], hw[2], hw[3]));
  }
  den += swap_halves_f32(den);
  __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0) lgkmcnt(0): this wave's plane loads have landed
  __syncthreads();                      // ... and every other wave's
  inv_l = 1.f / den;

  // ---- U^T = P^T phi'(Q)^T, then each row e times its factor (rows e >= 64 sit in v1: out_off(e - 64, c) has the
  // same swizzle bits as out_off(e, c))
  v16f acc[4];
#pragma unroll
  for (int et = 0; et < 4; ++et) {
    acc[et] = (v16f){};
    const int e = 32 * et + lr;
    const unsigned char* hp = et < 2 ? v0 : v1;
    const int eh = et < 2 ? e : e - 64;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const v8h a = *(const v8h*)(hp + out_off(eh, 16 * s + 8 * g));
      acc[et] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bq16[s], acc[et], 0, 0, 0);
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 f = *(const float4*)(s_f + 32 * et + 8 * r4 + 4 * g);
      acc[et][4 * r4] *= f.x;
      acc[et][4 * r4 + 1] *= f.y;
      acc[et][4 * r4 + 2] *= f.z;
      acc[et][4 * r4 + 3] *= f.w;
    }
  }
  __syncthreads();  // every wave is done with the plane
  {  // W_p^T (already in the plane layout) into the V slots: 32 loads of 1 KB
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wpt), (short)0, kD * kD * 2, 0x00020000);
#pragma unroll
    for (int i = 0; i < 32 / NW; ++i) {
      const int k = w + NW * i;
      unsigned char* dst = k < 16 ? v0 + k * 1024 : v1 + (k - 16) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)dst, 16, l * 16,
                                               k * 1024, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(7 << 4);
  }
  __syncthreads();

  // ---- O^T = W_p^T U^T: B operand slot (g, i) of step s2 is e = 16 s2 + 8(i/4) + 4g + i%4, i.e. accumulator
  // register 8(s2%2) + i of tile s2/2 in this lane; W_p^T rows hold e in the matching permuted order.
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
      const int f = 32 * ft + lr;
      const v8bf a = *(const v8bf*)((ft < 2 ? v0 : v1) + out_off(ft < 2 ? f : f - 64, 16 * s2 + 8 * g));
      acc2[ft] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bhi, acc2[ft], 0, 0, 0);
      acc2[ft] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, blo, acc2[ft], 0, 0, 0);
    }
  }
}

// G: one INT8 scale per 32 tokens of Q and of K (q_scale and k_scale hold ceil(N / 32) values per (b, h)): each
// wave's 32 rows are one group of Q, and each 32-key score tile one group of K.
template <int NW, bool G>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void k3_attn(
    const int8_t* __restrict__ q8, const int8_t* __restrict__ k8, const unsigned char* __restrict__ vt,
    const float* __restrict__ qs, const float* __restrict__ ks, const int32_t* __restrict__ kn2,
    const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ qraw, const unsigned char* __restrict__ plane16,
    const unsigned char* __restrict__ aux16, const uint16_t* __restrict__ wpt,
    float* __restrict__ o_lin, uint16_t* __restrict__ out, int N, int n_qb, int n_kb, int topk, float c0,
    int total) {
  constexpr int BLKQ = 32 * NW;
  // two rings of three slots: K codes (64 keys x 128 B) and V^T images (128 x 64 bf16). Each slot is its own
  // LDS object so that the compiler can tell the slot being filled from the slots being read.
  __shared__ __attribute__((aligned(1024))) unsigned char s_k0[64 * 128], s_k1[64 * 128], s_k2[64 * 128];
  __shared__ __attribute__((aligned(1024))) unsigned char s_v0[128 * 128], s_v1[128 * 128], s_v2[128 * 128];
  // the selection list as the steady loop consumes it: block index and scale product cq * k_scale per entry
  // (lists of up to kListCap entries, padded with four copies of the last index; longer lists are read through
  // scalar loads)
  __shared__ int s_lj[kListCap + 4];
  __shared__ float s_lc[kListCap];

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
      koff[tt][s] = kr * 128 + (((2 * s + g) ^ swz32(kr)) << 4);
    }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int vr = 32 * ct + lr;
      voff[ct][s] = vr * 128 + (((2 * s + g) ^ swz32(vr)) << 4);
    }
  const int n_g = (N + 31) / 32;
  // this wave's query scale times sm_scale * log2(e); cq_max over the workgroup's waves decides the exponent form
  // for all of them
  float cq, cq_max;
  if (G) {
    cq = qs[(size_t)bh * n_g + min(I * NW + w, n_g - 1)] * c0;
    cq_max = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) cq_max = fmaxf(cq_max, qs[(size_t)bh * n_g + min(I * NW + k, n_g - 1)] * c0);
  } else {
    cq = cq_max = qs[(size_t)bh * n_qb + I] * c0;
  }
  // The selection list and the key scales do not change during this kernel: reading them through the constant
  // address space lets the uniform reads use scalar loads, which do not count against the vector-memory
  // counter that the tile ring waits on.
  typedef __attribute__((address_space(4))) const int32_t c_i32;
  typedef __attribute__((address_space(4))) const float c_f32;
  c_i32* irow = (c_i32*)(idx + ((size_t)bh * n_qb + I) * topk);
  // descriptors over this (b, h)'s K codes and V^T images; every tile offset stays below their sizes (rows past
  // a ragged end re-read the last valid row)
  const __amdgpu_buffer_rsrc_t rk = slab_rsrc(k8 + (size_t)bh * N * kD, (uint32_t)N * kD);
  const __amdgpu_buffer_rsrc_t rv = slab_rsrc(vt + (size_t)bh * n_kb * 16384, (uint32_t)n_kb * 16384u);
  c_f32* ksrow = (c_f32*)(ks + (size_t)bh * (G ? n_g : n_kb));
  c_i32* knrow = (c_i32*)(kn2 + (size_t)bh * (G ? n_g : n_kb));
  const int last_kb = n_kb - 1;
  const int nv_last = N - last_kb * kBlkK;  // valid keys of the last key block (64 unless ragged)
  const StageOffsets<NW> so_full = stage_offsets<NW>(kBlkK);
  const StageOffsets<NW> so_last = stage_offsets<NW>(nv_last);

  v16f o[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) o[ct] = (v16f){};
  float m_run = -INFINITY, l_run = 0.f;

  auto blk = [&](int j) { return min(max(irow[j], 0), last_kb); };
  // the codes of the first key of the first selected block (the bounded shift's lower bound), in the lane's half
  // of the channels as bq holds them; loaded here so that their latency overlaps the list pass below
  const int J0 = topk > 0 ? blk(0) : 0;
  v4i kk0[4];
  {
    const int8_t* k0row = k8 + ((size_t)bh * N + (size_t)J0 * kBlkK) * kD;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) kk0[s4] = *(const v4i*)(k0row + 32 * s4 + 16 * g);
  }
  // key scales of block J for score tiles 0 and 1 (G: its two 32-key groups; the second group of a last block
  // that ends inside its first half does not exist and is clamped, its keys are masked anyway)
  auto kscale = [&](int J) -> float2 {
    if (G) return make_float2(ksrow[2 * J], ksrow[min(2 * J + 1, n_g - 1)]);
    const float k1 = ksrow[J];
    return make_float2(k1, k1);
  };
  // the largest code-row norm under each of those scales
  auto knorm = [&](int J) -> float2 {
    if (G) return make_float2(sqrtf((float)knrow[2 * J]), sqrtf((float)knrow[min(2 * J + 1, n_g - 1)]));
    const float n1 = sqrtf((float)knrow[J]);
    return make_float2(n1, n1);
  };
  auto stage = [&](int j, int buf) {
    const int J = blk(j);
    attn_stage<NW, G ? 1 : 0>(rk, rv, J, J == last_kb ? so_last : so_full,
                   buf ? s_k1 : s_k0, buf ? s_v1 : s_v0);
  };
  auto sync = [&]() {
    wait_vmem_all();
    __syncthreads();
  };
  if (topk > 0) {
    // Only the last key block can be ragged. Ascending lists hold it last, so every iteration but the last
    // runs the full-block body; a caller-given list that places it elsewhere takes the generic loop.
    // One pass over the list, a lane per entry: the largest key scale and whether the ragged block occurs
    // before the end.
    // Wave 0 also writes the list to LDS when it fits.
    const bool has_ragged = nv_last != kBlkK;
    // (G: the list keeps the two raw key scales per entry, in half the entries; each wave multiplies by its cq)
    const bool listed = topk <= (G ? kListCap / 2 : kListCap);
    float kmax = 0.f, kbn = 0.f;  // (kbn: the largest scale x code-row norm of the listed blocks)
    bool early_ragged = false;
    for (int j = l; j < topk; j += 64) {
      const int J = blk(j);
      const float2 kv = kscale(J);
      kmax = fmaxf(kmax, fmaxf(kv.x, kv.y));
      const float2 kn = knorm(J);
      kbn = fmaxf(kbn, fmaxf(kv.x * kn.x, kv.y * kn.y));
      early_ragged |= has_ragged && j < topk - 1 && J == last_kb;
      if (listed && w == 0) {
        s_lj[j] = J;
        if (G)
          ((float2*)s_lc)[j] = kv;
        else
          s_lc[j] = cq * kv.x;
      }
    }
    if (listed && w == 0 && l < 4) s_lj[topk + l] = blk(topk - 1);
    kmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max_f32(kmax))));
    kbn = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max_f32(kbn))));
    // the bound of the row's scores in exponent units (bounded shift): |codeQ_i| * cq * kbn (Cauchy-Schwarz),
    // rounded up (the two lane halves hold 64 codes each of the row; the squared norm is exact)
    int qn2 = 0;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int e = 0; e < 4; ++e) qn2 = __builtin_amdgcn_sdot4(bq[s4][e], bq[s4][e], qn2, false);
    qn2 += swap_halves_i32(qn2);
    const float brow = sqrtf((float)qn2) * cq * kbn * (1.f + 0x1p-16f);
    // a lower bound of the row's max: its score against the first key of its first selected block
    int s0 = 0;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int e = 0; e < 4; ++e) s0 = __builtin_amdgcn_sdot4(bq[s4][e], kk0[s4][e], s0, false);
    s0 += swap_halves_i32(s0);
    const float mlow = (float)s0 * (cq * kscale(J0).x);
    // per wave (the two paths meet the same barriers); lists of one block keep the running max
    const bool bounded = topk > 1 && __ballot(!(brow - mlow <= kBoundGap)) == 0;  // a NaN fails the test too
    if (bounded) m_run = brow - kBoundTop;
    const bool elsewhere = __ballot(early_ragged) != 0;
    const bool tail_ragged = has_ragged && blk(topk - 1) == last_kb;
    // one-instruction exponent argument when every block's scale product is below 2^-10 (see attn_exp_pair)
    const bool fast = cq_max * kmax < 0x1p-10f;
    v16i scur[2], snext[2];
    using T = AttnTile<NW>;
    using i0 = std::integral_constant<int, 0>;
    using i1 = std::integral_constant<int, 1>;
    using i2 = std::integral_constant<int, 2>;
    // K codes and V^T images travel in separate three-slot rings, each tile issued two iterations before its
    // use: iteration j reads K[j+1] (scores of the next block) and V[j], and issues K[j+3] and V[j+2] into the
    // slots that K[j] and V[j-1] leave free. The slots are distinct restrict-qualified pointers so that the
    // compiler can tell the loads in flight from the LDS reads of the current tiles.
    // With the list in LDS (L), iteration j takes J[j+3] and the scale product of block j from LDS reads issued
    // one iteration earlier, which the ring's barrier wait has already completed: the steady loop then has no
    // scalar-memory waits (those would also drain the LDS operand reads in flight).
    auto ring = [&](auto fastc, auto listc, auto boundc, unsigned char* __restrict__ k0,
                    unsigned char* __restrict__ k1, unsigned char* __restrict__ k2, unsigned char* __restrict__ v0,
                    unsigned char* __restrict__ v1, unsigned char* __restrict__ v2) {
      constexpr bool F = decltype(fastc)::value;
      constexpr bool L = decltype(listc)::value;
      constexpr bool BD = decltype(boundc)::value;
      unsigned char* const ks[3] = {k0, k1, k2};
      unsigned char* const vs[3] = {v0, v1, v2};
      // K tiles use the full-block offsets even for a ragged last block: its rows past N lie beyond the
      // descriptor's range, so those loads return zeros without touching memory, and the ragged pass masks the
      // keys anyway
      auto put_kJ = [&](int J, unsigned char* dst) {
        stage_k<NW, G ? 1 : 0>(rk, (uint32_t)J * (kBlkK * kD), so_full, dst);
      };
      auto put_vJ = [&](int J, unsigned char* dst) { stage_v<NW>(rv, (uint32_t)J * 16384u, dst); };
      auto put_k = [&](int j, unsigned char* dst) { put_kJ(blk(j), dst); };
      auto put_v = [&](int j, unsigned char* dst) { put_vJ(blk(j), dst); };
      put_k(0, k0);
      if (topk > 1) put_k(1, k1);
      if (topk > 2) put_k(2, k2);
      put_v(0, v0);
      if (topk > 1) put_v(1, v1);
      ring_sync<0>();
      attn_scores(k0, bq, koff, scur);
      auto pick = [&](int r, unsigned char* x0, unsigned char* x1, unsigned char* x2) {
        return r == 0 ? x0 : r == 1 ? x1 : x2;
      };
      // Iteration j < topk - 1 waits for K[j+1] and V[j], issued two iterations back (the loads of iteration
      // j-1 may stay in flight), issues K[j+3] and V[j+2], then runs block j with the scores of block j+1.
      // Steady state, ring phase P = j % 3 known at compile time, both tiles issued:
      // (L: lj holds J[j+3] and lc the scale product of block j (G: the two key scales of block j), both as
      // read from LDS; jv = J[j+2])
      int lj = 0, jv = 0;
      float2 lc = make_float2(0.f, 0.f);
      auto list_c = [&](int j) { return G ? ((const float2*)s_lc)[j] : make_float2(s_lc[j], 0.f); };
      if constexpr (L) {
        lj = s_lj[3];
        lc = list_c(0);
        jv = __builtin_amdgcn_readfirstlane(s_lj[2]);
      }
      // scale products of block j for tiles 0 and 1, from the scalar-load path
      auto cpair = [&](int J, float& ca, float& cb) {
        const float2 kv = kscale(J);
        ca = cq * kv.x;
        cb = G ? cq * kv.y : ca;
      };
      auto iter_full = [&](int j, auto ph) {
        constexpr int P = decltype(ph)::value;
        ring_sync<T::KPW + T::VPW>();
        float c, c1;
        if constexpr (L) {
          const int J3 = __builtin_amdgcn_readfirstlane(lj);
          if (G) {
            c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cq * lc.x)));
            c1 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cq * lc.y)));
          } else {
            c1 = c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(lc.x)));
          }
          put_kJ(J3, ks[P]);
          put_vJ(jv, vs[(P + 2) % 3]);
          lj = s_lj[j + 4];
          lc = list_c(j + 1);
          jv = J3;
        } else {
          put_k(j + 3, ks[P]);
          put_v(j + 2, vs[(P + 2) % 3]);
          cpair(blk(j), c, c1);
        }
        attn_iter<false, true, F, G, BD>(ks[(P + 1) % 3], vs[P], bq, koff, voff, c, c1, kBlkK, g, o, m_run, l_run,
                                     scur, snext);
        scur[0] = snext[0];
        scur[1] = snext[1];
      };
      // the last few iterations before the final block: slots picked at run time, tiles issued while they exist
      auto iter_tail = [&](int j) {
        const int P = j % 3;
        if (j + 2 < topk)
          ring_sync<T::KPW + T::VPW>();
        else
          ring_sync<T::VPW>();
        if (j + 3 < topk) put_k(j + 3, pick(P, k0, k1, k2));
        if (j + 2 < topk) put_v(j + 2, pick(P == 0 ? 2 : P - 1, v0, v1, v2));
        float c, c1;
        cpair(blk(j), c, c1);
        attn_iter<false, true, F, G, BD>(pick(P == 2 ? 0 : P + 1, k0, k1, k2), pick(P, v0, v1, v2), bq, koff, voff, c,
                                     c1, kBlkK, g, o, m_run, l_run, scur, snext);
        scur[0] = snext[0];
        scur[1] = snext[1];
      };
      int j = 0;
      for (; j + 5 < topk; j += 3) {
        iter_full(j, i0{});
        iter_full(j + 1, i1{});
        iter_full(j + 2, i2{});
      }
      for (; j < topk - 1; ++j) iter_tail(j);
      // last block (j == topk - 1), no successor
      ring_sync<0>();
      const int ph = j % 3;
      unsigned char* const vl = ph == 0 ? v0 : ph == 1 ? v1 : v2;
      float c, c1;
      cpair(tail_ragged ? last_kb : blk(j), c, c1);
      if (tail_ragged)
        attn_iter<true, false, F, G, BD>(nullptr, vl, bq, koff, voff, c, c1, nv_last, g, o, m_run, l_run, scur,
                                         snext);
      else
        attn_iter<false, false, F, G, BD>(nullptr, vl, bq, koff, voff, c, c1, kBlkK, g, o, m_run, l_run, scur,
                                          snext);
    };
    if (elsewhere) {
      stage(0, 0);
      sync();
      for (int j = 0; j < topk; ++j) {
        const int buf = j & 1;
        if (j + 1 < topk) stage(j + 1, buf ^ 1);
        const int J = blk(j);
        const float2 kv = kscale(J);
        attn_scores(buf ? s_k1 : s_k0, bq, koff, scur);
        attn_iter<true, false, false, G>(nullptr, buf ? s_v1 : s_v0, bq, koff, voff, cq * kv.x, cq * kv.y,
                                         min(kBlkK, N - J * kBlkK), g, o, m_run, l_run, scur, snext);
        sync();
      }
    } else {
      auto with_bound = [&](auto fastc, auto listc) {
        if (bounded)
          ring(fastc, listc, std::true_type{}, s_k0, s_k1, s_k2, s_v0, s_v1, s_v2);
        else
          ring(fastc, listc, std::false_type{}, s_k0, s_k1, s_k2, s_v0, s_v1, s_v2);
      };
      if (fast) {
        if (listed)
          with_bound(std::true_type{}, std::true_type{});
        else
          with_bound(std::true_type{}, std::false_type{});
      } else {
        if (listed)
          with_bound(std::false_type{}, std::true_type{});
        else
          with_bound(std::false_type{}, std::false_type{});
      }
    }
  }

  const float lt = l_run + swap_halves_f32(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // the linear branch (rec16 given): O_l in the same register layout as O
  v16f ol[4];
  float inv_l = 0.f;
  if (plane16) lin_epilogue<NW>(qraw, plane16, aux16, wpt, bh, I, N, n_qb, s_k2, s_v0, s_v1, ol, inv_l);
  if (rok) {
    const size_t ro = ((size_t)bh * N + row) * kD;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int e0 = 32 * ct + 8 * r4 + 4 * g;
        float x0 = o[ct][4 * r4] * inv, x1 = o[ct][4 * r4 + 1] * inv;
        float x2 = o[ct][4 * r4 + 2] * inv, x3 = o[ct][4 * r4 + 3] * inv;
        if (plane16) {
          const float4 a = make_float4(ol[ct][4 * r4] * inv_l, ol[ct][4 * r4 + 1] * inv_l, ol[ct][4 * r4 + 2] * inv_l,
                                       ol[ct][4 * r4 + 3] * inv_l);
          if (o_lin) *(float4*)(o_lin + ro + e0) = a;
          x0 += a.x; x1 += a.y; x2 += a.z; x3 += a.w;
        }
        *(uint2*)(out + ro + e0) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
      }
  }
}

hipError_t launch_attn(const Plan& p, const uint16_t* q, uint16_t* out, hipStream_t s) {
  const int total = p.BH * p.n_qb;
  const float c0 = p.sm_scale * 1.4426950408889634f;  // log2(e): scores enter exp2
  const bool lin = p.linear && p.topk < p.n_kb;
  const unsigned char* pl16 = lin ? p.plane16 : nullptr;
  float* olin = lin ? p.o_lin : nullptr;  // optional export of the linear branch's output
#define SAGESLA_ATTN(NWV, G)                                                                                     \
  hipLaunchKernelGGL((k3_attn<NWV, G>), dim3(total), dim3(64 * NWV), 0, s, p.q_i8, p.k_i8, p.v_img, p.q_scale,     \
                     p.k_scale, p.k_norm2, p.block_idx, q, pl16, p.aux16, p.wpt, olin, out, p.N, p.n_qb, p.n_kb,    \
                     p.topk, c0, total)
  if (p.blk_q == 128) {
    if (p.group32) SAGESLA_ATTN(4, true); else SAGESLA_ATTN(4, false);
  } else {
    if (p.group32) SAGESLA_ATTN(2, true); else SAGESLA_ATTN(2, false);
  }
#undef SAGESLA_ATTN
  return hipGetLastError();
}

}  // namespace sagesla
