"""W8A8 block-quantized linear layer on MI355X (gfx950): thin Python binding of the w8a8_* entry points of
libsagesla.so (include/w8a8.h).

Y = X W^T + b with 8-bit codes and one fp32 scale per 128×128 block of X and of W. Every step runs in the
library's HIP kernels; this module only checks tensor shapes and marshals pointers. There is no CPU fallback.
"""
from __future__ import annotations

from . import _check, _ptr, _stream, load

__all__ = ["quantize", "gemm", "linear", "workspace_bytes", "n_blocks"]


def n_blocks(n: int) -> int:
    return -(-n // 128)


def _need(t, name, dtype, shape=None):
    import torch
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    del torch


def quantize(x, clip: float = 1.0, codes=None, scales=None):
    """128×128 block quantizer: x bf16 [R, C] (C a multiple of 128) -> (codes int8 [R, C],
    scales fp32 [ceil(R / 128), C / 128]). clip in (0, 1]: threshold = clip * absmax of each block."""
    import torch
    _need(x, "x", torch.bfloat16)
    R, C = x.shape
    if codes is None:
        codes = torch.empty(R, C, dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty(n_blocks(R), C // 128 if C % 128 == 0 else 1, dtype=torch.float32, device=x.device)
    _check(load().w8a8_quantize(x.data_ptr(), R, C, float(clip), codes.data_ptr(), scales.data_ptr(),
                                _stream(x.device)), "w8a8_quantize")
    return codes, scales


def gemm(x_i8, x_scale, w_i8, w_scale, bias=None, out=None):
    """Block-scaled INT8 product from codes and scales: returns bf16 [M, N] = dequantized X W^T + bias."""
    import torch
    M, K = x_i8.shape
    N = w_i8.shape[0]
    _need(x_i8, "x_i8", torch.int8)
    _need(w_i8, "w_i8", torch.int8, (N, K))
    _need(x_scale, "x_scale", torch.float32, (n_blocks(M), K // 128))
    _need(w_scale, "w_scale", torch.float32, (n_blocks(N), K // 128))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,))
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=x_i8.device)
    _need(out, "out", torch.bfloat16, (M, N))
    _check(load().w8a8_gemm(x_i8.data_ptr(), x_scale.data_ptr(), w_i8.data_ptr(), w_scale.data_ptr(), _ptr(bias),
                            out.data_ptr(), M, N, K, _stream(x_i8.device)), "w8a8_gemm")
    return out


def workspace_bytes(M: int, K: int) -> int:
    return load().w8a8_workspace_bytes(M, K)


def linear(x, w_i8, w_scale, bias=None, clip: float = 1.0, out=None, workspace=None):
    """The whole layer: x bf16 [M, K] is quantized at call time (clip ratio `clip`) and multiplied with the
    pre-quantized weights (w_i8 int8 [N, K], w_scale fp32 [N / 128, K / 128] from quantize(W))."""
    import torch
    M, K = x.shape
    N = w_i8.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(w_i8, "w_i8", torch.int8, (N, K))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,))
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (M, N))
    need = workspace_bytes(M, K)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check(load().w8a8_linear(x.data_ptr(), w_i8.data_ptr(), w_scale.data_ptr(), _ptr(bias), out.data_ptr(), M, N,
                              K, float(clip), workspace.data_ptr(), workspace.numel(), _stream(x.device)),
           "w8a8_linear")
    return out
