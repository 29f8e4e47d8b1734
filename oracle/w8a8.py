"""Plain, slow fp64 CPU oracle of the W8A8 block-quantized linear layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this module: only the
tests and the benchmark's CPU-baseline leg use it. It shares no code, constant or helper with the HIP
library (nor with the attention oracle); both sides only consume the same seeded inputs.

What is computed, and where the pages say so
--------------------------------------------
  [TD-news]    "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn/news/1185.html), §三(四) item 1
               (W8A8 block quantization): 1) the weight matrix of a linear layer is cut into independent
               128×128 blocks, each with its own quantization parameters; 2) activations are quantized
               dynamically from statistics of the layer's input at run time, with clipping that bounds the
               extreme values.
  [TD-release] chooseai.net news 1890 (the TurboDiffusion release), the list of the four techniques: the
               linear-layer acceleration quantizes both the parameters and the activations to 8 bits in
               128×128 blocks.

Readings where the pages stop (the plainest ones the rest supports):
  * The layer is Y = X W^T + b with X [M, K] (tokens × input features), W [N, K] (output × input features,
    the usual weight layout), b [N] optional.
  * Both matrices are cut into blocks of 128 rows × 128 columns of their own layout; the column (input
    feature) blocking is shared, so k-block kb pairs block (mb, kb) of X with block (nb, kb) of W. A ragged
    last row block of X holds only its valid rows; N and K are multiples of 128.
  * Per block: t = fp32(alpha * absmax), s = fp32(t / 127), code = clamp(round-half-even(fp32(x / s)), -127,
    127). alpha in (0, 1] is the clip ratio: values beyond the threshold t saturate at +-127. Weights use
    alpha = 1 (no clipping); activations take alpha from the caller. A block whose s is 0 (absmax 0, or a
    threshold so small that s underflows) gets s = 0 and all-zero codes.
  * The product: Y[m, n] = sum over k-blocks kb of s_x(mb, kb) * s_w(nb, kb) * P_kb[m, n] + b[n], with
    P_kb = sum over the 128 columns of the k-block of code_x * code_w (an exact integer).
The fp32(.) points are single IEEE operations on fp32/bf16 operands; computing each in fp64 and rounding to
fp32 gives the correctly rounded fp32 result (53 >= 2*24 + 2; Figueroa, "When is double rounding innocuous?",
1995). Everything else is fp64.
"""
from __future__ import annotations

import numpy as np

__all__ = ["BLK", "n_blocks", "quantize_blocks", "dequantize_blocks", "block_gemm", "linear", "abs_terms"]

BLK = 128
QMAX = 127.0


def n_blocks(n: int, blk: int = BLK) -> int:
    return -(-n // blk)


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def quantize_blocks(X: np.ndarray, clip: float = 1.0):
    """Block INT8 quantizer of [TD-news] §三(四) item 1 (128×128 blocks; clipping for activations).

    X [R, C] with C a multiple of 128. Returns (codes int8 [R, C], scales float64 holding fp32 values
    [ceil(R / 128), C / 128])."""
    X = np.asarray(X, dtype=np.float64)
    R, C = X.shape
    if C % BLK:
        raise ValueError("the column count must be a multiple of 128")
    alpha = float(np.float32(clip))
    if not (0.0 < alpha <= 1.0):
        raise ValueError("clip ratio must lie in (0, 1]")
    codes = np.zeros((R, C), dtype=np.int8)
    scales = np.zeros((n_blocks(R), C // BLK), dtype=np.float64)
    for mb in range(n_blocks(R)):
        r0, r1 = mb * BLK, min(R, (mb + 1) * BLK)
        for kb in range(C // BLK):
            blk = X[r0:r1, kb * BLK:(kb + 1) * BLK]
            amax = float(np.max(np.abs(blk)))
            if amax == 0.0:
                continue
            t = float(_f32(alpha * amax))
            s = float(_f32(t / QMAX))
            if s == 0.0:  # the threshold underflowed: treated as an all-zero block
                continue
            q = np.rint(_f32(blk / s))  # fp32 quotient, then round half to even
            codes[r0:r1, kb * BLK:(kb + 1) * BLK] = np.clip(q, -QMAX, QMAX).astype(np.int8)
            scales[mb, kb] = s
    return codes, scales


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code * s of each element's block (fp64)."""
    codes = np.asarray(codes, dtype=np.float64)
    R, C = codes.shape
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), BLK, axis=0)[:R], BLK, axis=1)[:, :C]
    return codes * s


def block_gemm(xq, xs, wq, ws, bias=None) -> np.ndarray:
    """Y[m, n] = sum_kb s_x(mb, kb) s_w(nb, kb) P_kb[m, n] + b[n] in fp64, P_kb the exact integer product of the
    codes over the columns of k-block kb (one int64 matmul per k-block)."""
    xq = np.asarray(xq, dtype=np.int64)
    wq = np.asarray(wq, dtype=np.int64)
    M, K = xq.shape
    N = wq.shape[0]
    Y = np.zeros((M, N), dtype=np.float64)
    xs = np.asarray(xs, np.float64)
    ws = np.asarray(ws, np.float64)
    for kb in range(K // BLK):
        P = xq[:, kb * BLK:(kb + 1) * BLK] @ wq[:, kb * BLK:(kb + 1) * BLK].T  # exact
        cx = np.repeat(xs[:, kb], BLK)[:M]  # s_x of each row's block
        cw = np.repeat(ws[:, kb], BLK)[:N]  # s_w of each output column's block
        Y += (cx[:, None] * cw[None, :]) * P.astype(np.float64)
    if bias is not None:
        Y += np.asarray(bias, np.float64)[None, :]
    return Y


def abs_terms(xq, xs, wq, ws, bias=None) -> np.ndarray:
    """sum_kb |s_x s_w P_kb| + |b|: the magnitude that bounds the rounding error of any summation order."""
    xq = np.asarray(xq, dtype=np.int64)
    wq = np.asarray(wq, dtype=np.int64)
    M, K = xq.shape
    N = wq.shape[0]
    A = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // BLK):
        P = xq[:, kb * BLK:(kb + 1) * BLK] @ wq[:, kb * BLK:(kb + 1) * BLK].T
        cx = np.repeat(np.asarray(xs, np.float64)[:, kb], BLK)[:M]
        cw = np.repeat(np.asarray(ws, np.float64)[:, kb], BLK)[:N]
        A += np.abs((cx[:, None] * cw[None, :]) * P.astype(np.float64))
    if bias is not None:
        A += np.abs(np.asarray(bias, np.float64))[None, :]
    return A


def linear(X, W, bias=None, clip: float = 1.0):
    """The W8A8 linear layer: quantize W (no clipping) and X (clip ratio `clip`), then the block-scaled product.
    Returns (Y fp64 [M, N], (xq, xs), (wq, ws))."""
    xq, xs = quantize_blocks(X, clip)
    wq, ws = quantize_blocks(W, 1.0)
    return block_gemm(xq, xs, wq, ws, bias), (xq, xs), (wq, ws)
