// Helpers of the linear branch shared by the state kernels and the attention kernel's epilogue.
#pragma once

#include "device_common.h"

namespace sagesla {

// position of key/channel slot inside a 16-group such that the MFMA 32x32x16 lane (half g, slot i) reads
// 8 consecutive positions: slot (g, i) <-> index 8*(i/4) + 4*g + (i%4); position 8*g + 4*(i/4) + (i%4).
__device__ __forceinline__ int slot_pos16(int off) {  // off = index within the 16-group
  return (off & 3) | ((off & 4) << 1) | ((off & 8) >> 1);
}

// A [128][128] bf16 plane as the linear-branch output keeps it in LDS (and the remaining state is stored): rows
// of 256 B, 16-byte chunks XOR-swizzled by row. Byte offset of (row, col):
__device__ __forceinline__ int out_off(int e, int c) { return e * 256 + ((((c >> 3) ^ e) & 15) << 4) + ((c & 7) << 1); }

// phi(x) = elu(x) + 1: x + 1 for x > 0, e^x otherwise (hardware exp2 of x log2(e); the values then enter the
// MFMAs as hi + lo bf16 pairs, ~16 significant bits)
__device__ __forceinline__ float phi_f(float x) {
  return x > 0.f ? x + 1.f : __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// The forward's per-block state table is fp16 with one power of two per key block: entries x * 2^(15 - k) for the
// block's largest magnitude M < 2^k, and the block exponent e_J = k - 15; an all-zero block has e_J = kExpZero.
constexpr int kExpZero = -100000;

// two fp32 values -> bf16 pairs hi = bf16(x) and lo = bf16(x - hi), packed as (x0, x1)
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(x0, x1);
  lo = pack_bf16x2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
}

}  // namespace sagesla
