/*
 * w8a8.h — C ABI of the W8A8 block-quantized linear layer for AMD Instinct MI355X (gfx950), in the same
 * library as the SageSLA attention (libsagesla.so) and sharing its status codes.
 *
 * The linear layers either side of a video-DiT attention run with 8-bit weights and 8-bit activations:
 *   [TD-news]    "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn), §三(四) item 1: weights in
 *                independent 128×128 blocks with their own quantization parameters; activations quantized
 *                dynamically at run time, with clipping of extreme values;
 *   [TD-release] chooseai.net news 1890 (the TurboDiffusion release), list of the four techniques: parameters
 *                and activations of the linear layers both in 8-bit 128×128 blocks.
 *
 * The layer: Y = X W^T + b, X [M][K] bf16 (tokens × input features), W [N][K] bf16 (output × input features),
 * b [N] bf16 (optional), Y [M][N] bf16. N and K must be multiples of 128; M is free (the last row block of X
 * holds only the remaining rows).
 *
 * Quantizer (both matrices, blocks of 128 rows × 128 columns of their own layout, block (rb, cb) row-major):
 *   t = fp32(clip * absmax), s = fp32(t / 127), code = clamp(round-half-even(fp32(x / s)), -127, 127);
 *   a block whose s is 0 (all-zero block) gets all-zero codes. Values beyond t saturate at +-127. Weights are
 *   quantized once with clip = 1; activations at every call with the caller's clip ratio in (0, 1].
 * Product: Y[m][n] = bf16_rne( sum over k-blocks kb, ascending, in fp32 of fp32(s_x(mb, kb) * s_w(nb, kb)) * P_kb
 *   + b[n] ), P_kb = the exact integer sum over the 128 columns of k-block kb of code_x * code_w; each step is
 *   one fused multiply-add of P_kb (exact in fp32) into the running sum.
 *
 * Conventions: every data pointer is a device pointer owned by the caller and 16-byte aligned (workspace:
 * 256-byte aligned); calls are asynchronous on `stream` (a hipStream_t as void*; NULL is the null stream);
 * parameters are checked on the host before any launch and nothing is launched on an error; results are
 * deterministic; inputs must be finite. Two calls that share output or workspace buffers must not overlap.
 * Limits (else SAGESLA_E_UNSUPPORTED): rows * cols < 2^31 for each matrix, K <= 32768, M and N <= 2^24.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#include "sagesla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Block quantizer ([TD-news] §三(四) item 1). x: bf16 [rows][cols], cols a multiple of 128. Writes
   codes [rows][cols] (int8) and scales [ceil(rows / 128)][cols / 128] (fp32). clip in (0, 1] (1 = none).
   Codes and scales are bit-exact functions of x and clip. SAGESLA_E_SHAPE for rows < 1, cols < 1 or clip
   outside (0, 1]; SAGESLA_E_UNSUPPORTED for cols not a multiple of 128 or sizes past the limits. */
sagesla_status w8a8_quantize(const void* x, int32_t rows, int32_t cols, float clip, int8_t* codes,
                             float* scales, void* stream);

/* Block-scaled INT8 product (the formula above) from codes and scales as w8a8_quantize writes them:
   x_i8 [M][K], x_scale [ceil(M/128)][K/128], w_i8 [N][K], w_scale [N/128][K/128], bias bf16 [N] or NULL,
   y bf16 [M][N]. */
sagesla_status w8a8_gemm(const int8_t* x_i8, const float* x_scale, const int8_t* w_i8, const float* w_scale,
                         const void* bias, void* y, int32_t M, int32_t N, int32_t K, void* stream);

/* Bytes of workspace w8a8_linear needs (activation codes and scales); 0 for invalid sizes. Host only. */
size_t w8a8_workspace_bytes(int32_t M, int32_t K);

/* The whole layer: quantizes x (bf16 [M][K]) with clip ratio `clip` into the workspace, then runs w8a8_gemm
   with the pre-quantized weights. */
sagesla_status w8a8_linear(const void* x, const int8_t* w_i8, const float* w_scale, const void* bias, void* y,
                           int32_t M, int32_t N, int32_t K, float clip, void* workspace, size_t workspace_bytes,
                           void* stream);

#ifdef __cplusplus
}
#endif
#endif /* W8A8_H */
