// Practical peak of the matrix cores: a loop of independent MFMAs with no memory traffic, timed by the caller.
// Measurement tooling for the benchmark (libsagesla_probe.so), not part of the attention library.
//
// Each wave keeps four independent accumulator chains (so no MFMA waits for the previous one's result) and
// issues 4 * iters MFMAs of one kind:
//   kind 0: v_mfma_i32_32x32x32_i8   (32*32*32 multiply-adds = 65536 INT8 ops each)
//   kind 1: v_mfma_f32_32x32x16_bf16 (32*32*16 multiply-adds = 32768 flops each)
//   kind 2: v_mfma_f32_32x32x16_f16
// The operands depend on the lane and a run-time seed, and every accumulator is written out, so nothing is
// folded away. out must hold gridDim.x * blockDim.x floats.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(256) void probe_mfma(float* __restrict__ out, int iters, int seed) {
  const int t = threadIdx.x;
  const int x = (t * 2654435761u + seed) & 0x3F3F3F3F;  // small values: no int overflow, finite floats
  float r = 0.f;
  if constexpr (KIND == 0) {
    const v4i a = {x, x ^ 0x01010101, x ^ 0x02020202, x ^ 0x03030303};
    const v4i b = {x ^ 0x04040404, x, x ^ 0x05050505, x ^ 0x06060606};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) r += (float)(c0[k] ^ c1[k] ^ c2[k] ^ c3[k]);
  } else {
    typedef typename std::conditional<KIND == 1, v8bf, v8h>::type V;
    typedef typename std::conditional<KIND == 1, __bf16, _Float16>::type E;
    V a, b;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[k] = (E)(float)((x >> k) & 7) * (E)0.125f;
      b[k] = (E)(float)((x >> (k + 8)) & 7) * (E)0.125f;
    }
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      if constexpr (KIND == 1) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
      } else {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c3, 0, 0, 0);
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) r += c0[k] + c1[k] + c2[k] + c3[k];
  }
  out[blockIdx.x * blockDim.x + t] = r;
}

}  // namespace

// Launches `blocks` workgroups of 256 threads (4 waves) on stream; returns the hipError_t of the launch.
extern "C" int sagesla_probe_mfma(int kind, int blocks, int iters, int seed, float* out, void* stream) {
  if (kind < 0 || kind > 2 || blocks < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
  const hipStream_t s = (hipStream_t)stream;
  if (kind == 0) hipLaunchKernelGGL(probe_mfma<0>, dim3(blocks), dim3(256), 0, s, out, iters, seed);
  if (kind == 1) hipLaunchKernelGGL(probe_mfma<1>, dim3(blocks), dim3(256), 0, s, out, iters, seed);
  if (kind == 2) hipLaunchKernelGGL(probe_mfma<2>, dim3(blocks), dim3(256), 0, s, out, iters, seed);
  return (int)hipGetLastError();
}
