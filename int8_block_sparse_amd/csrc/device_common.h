// Small device helpers for the gfx950 kernels (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sagesla {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  v2f x = {a, b};
  v2h y = __builtin_convertvector(x, v2h);
  return __builtin_bit_cast(uint32_t, y);
}

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  v2f x = {a, b};
  v2bf y = __builtin_convertvector(x, v2bf);
  return __builtin_bit_cast(uint32_t, y);
}

// fp32 -> (hi, lo) bf16 split: hi = bf16(x), lo = bf16(x - hi); hi + lo carries ~16 significant bits
__device__ __forceinline__ void split_bf16(float x, float& hi, float& lo) {
  uint32_t h = pack_bf16x2(x, 0.f) & 0xffffu;
  hi = __uint_as_float(h << 16);
  lo = x - hi;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// value of lane (l ^ 32). v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes 0..31 of
// its second: with both operands = v, the first result holds the other half's value in lanes 32..63 and the
// second result holds it in lanes 0..31.
__device__ __forceinline__ int swap_halves_i32(int v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float swap_halves_f32(float v) {
  return __int_as_float(swap_halves_i32(__float_as_int(v)));
}
// max over lanes l and l ^ 32, on every lane: the swap leaves one half's value in both halves of each result
__device__ __forceinline__ int max_halves_i32(int v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((int)r[0], (int)r[1]);
}

// Key order inside each group of 16 keys of a V^T row in LDS: the bf16 MFMA lane half g, slot i (0..7) must
// find key 8*(i/4) + 4*g + (i%4) at position 8*g + i, i.e. the middle two groups of 4 keys trade places.
__device__ __forceinline__ int key_pos16(int off) { return (off & 3) | ((off & 4) << 1) | ((off & 8) >> 1); }

// XOR swizzle of the 16-byte chunk index inside a 128-byte LDS row, so that both 8 consecutive rows read at
// one chunk and rows 8 apart written at one chunk land in different banks.
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }
// The same pattern built from the low five row bits only, so that it repeats every 32 rows: operand reads of
// 32-row MFMA tiles at rows 32t + lane then differ from tile 0's by the constant 4096 * t, which the LDS
// instructions take as an immediate offset instead of a register per tile. Each read still touches 32 rows
// that share bit 5, where the two patterns differ by a constant XOR, so it stays conflict-free.
__device__ __forceinline__ int swz32(int row) { return (row ^ ((row >> 3) & 3)) & 7; }

// The INT8 code clamp(round-half-even(fp32(x / s)), -127, 127) of x for a scale s > 0 and r = fp32(1/s):
// q = fp32(x * r) differs from the correctly rounded quotient f = fp32(x / s) by at most 2.3e-5 when |q| < 128
// (two roundings of relative 2^-24 each on a value below 128.0001, plus f's own half ulp, at most 2^-17), less
// than the 2^-15 margin tested below. round(q) can
// differ from round(f) only if a half-integer lies within that distance of q, so such rare elements (and
// non-finite q) are recomputed with the IEEE division. When |q| >= 128 (only under clipping), |f| > 127.5 and
// both round to a value that the clamp takes to +-127; the check then also sends q to the division unless it
// happens to be near an integer, which changes nothing.
__device__ __forceinline__ int quant_code(float x, float s, float r) {
#pragma clang fp contract(off)
  const float qv = x * r;
  float c = rintf(qv);
  if (!(fabsf(qv - c) < 0.5f - 0x1p-15f)) c = rintf(x / s);
  c = fminf(fmaxf(c, -127.f), 127.f);
  return (int)c;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) | ((uint32_t)d << 24);
}

// Swizzled tiles of rows of 256 B (128 16-bit elements): the 16-byte chunk c of row r sits at chunk position
// c ^ tswz(r). Sixteen consecutive rows at one chunk fall on sixteen distinct positions (the row reads of an MFMA
// operand), and four rows from a multiple of 4 over four aligned chunks fall on sixteen distinct positions
// (transposing reads).
__device__ __forceinline__ int tswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// byte offset of the 8-byte unit that holds columns col .. col + 3 (col a multiple of 4) of row r
__device__ __forceinline__ int toff(int r, int col) { return r * 256 + (((col >> 3) ^ tswz(r)) << 4) + ((col & 4) << 1); }

// Operand of a 32x32x16 16-bit MFMA read down the columns of a swizzled tile: lane l holds tile column
// m0 + l % 32 at rows i0 + 8 (l / 32) .. + 7 (slot s = row i0 + 8 (l / 32) + s), the order of an operand read
// along a row. Two transposing reads (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives
// element i % 4 of the 8-byte units addressed by lanes 4 c + i / 4, c = 0..3.
__device__ __forceinline__ v8s tr_col_op(const unsigned char* t, int i0, int m0, int l) {
  const int j = l & 15;
  const int r = i0 + 8 * (l >> 5) + (j >> 2);
  const int col = m0 + 16 * ((l >> 4) & 1) + 4 * (j & 3);
  const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + toff(r, col)));
  const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + toff(r + 4, col)));
  return (v8s){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Map a flat workgroup id to a work item so that each XCD (ids are dealt round-robin over 8 XCDs) gets one
// contiguous range of work items: neighbouring query blocks of a head then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = id & 7, local = id >> 3;
  return x * q + (x < r ? x : r) + local;
}

}  // namespace sagesla
