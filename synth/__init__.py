"""Seeded synthetic inputs for the SageSLA attention forward.

The TurboDiffusion pages measure SageSLA inside real Wan2.1/2.2 video DiTs ("Turbo Diffusion：秒级生成与高清保真
的视频扩散技术突破", lanhy.cn, §五; "TurboDiffusion技术指南", blog.gitcode.com, speed table). Neither the models nor
their activations are available, so the workloads here are synthetic tensors with the shape of one attention
layer of those models (heads × tokens × head-dim on the latent token grid) and stated value distributions.

This module holds none of the method's arithmetic. It only draws tensors; the CPU oracle and the HIP library
both consume exactly what it returns.

Recipe (all draws from one torch.Generator seeded with ``seed``, in this order):
  * bias[H, D]  = 2 * N(0,1)          -- per-(head, channel) offset added to K so that K-mean smoothing matters
  * W_p[D, D]   = N(0,1) / sqrt(D)    -- the D×D projection applied to the linear-branch output
  * for each batch index b:
      - iid workloads:        Q, K, V ~ N(0,1) of shape [H, N, D]
      - structured workloads: field noise ~ N(0,1) of shape [H, D, T, Hh, Ww]; the field is that noise
        blurred by a Gaussian (sigma 2 tokens, radius 8, edge-including mirror at the borders) along each of
        the three grid axes and divided by its own standard deviation over the grid, so each (head, channel)
        field has unit variance; Q = field + 0.3 N(0,1), K = field + 0.3 N(0,1), V ~ N(0,1)
      - K += bias[h, :]
  * everything is drawn in fp32 and rounded once to bf16 (round-to-nearest-even).
Tokens of a grid are ordered frame-major: n = t*(Hh*Ww) + y*Ww + x.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import torch

__all__ = ["Workload", "WORKLOADS", "workload", "custom", "make", "topk_blocks", "n_blocks", "LinearWorkload",
           "LINEAR_WORKLOADS", "make_linear", "make_norm_weights", "NORM_EPS"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    grid: Optional[Tuple[int, int, int]]  # (T, Hh, Ww) latent token grid, or None for unstructured tokens
    blk_q: int
    blk_k: int
    topk_frac: float  # fraction of key blocks kept per query block (the --sla_topk value)
    linear: bool  # whether the elu+1 linear branch runs on the non-selected blocks
    structured: bool  # smooth spatio-temporal field shared by Q and K

    @property
    def n_qb(self) -> int:
        return n_blocks(self.N, self.blk_q)

    @property
    def n_kb(self) -> int:
        return n_blocks(self.N, self.blk_k)

    @property
    def topk(self) -> int:
        return topk_blocks(self.topk_frac, self.n_kb)

    @property
    def dense_equiv_ops(self) -> float:
        """4·B·H·N²·D: QKᵀ plus PV of dense attention, the yardstick for 'dense-equivalent' throughput."""
        return 4.0 * self.B * self.H * float(self.N) ** 2 * self.D


def n_blocks(n: int, blk: int) -> int:
    return (n + blk - 1) // blk


def topk_blocks(frac: float, n_kb: int) -> int:
    """Number of key blocks kept per query block for a kept fraction ``frac`` of ``n_kb`` blocks.

    The user guide's --sla_topk flag is a fraction (0.1 keeps 10%). It is turned into a block count by rounding
    half up, at least one block, and all blocks for frac >= 1.
    """
    if frac >= 1.0:
        return n_kb
    return max(1, int(math.floor(frac * n_kb + 0.5)))


# The five layer shapes: a tiny case, the 1.3B-480P layer dense and sparse, the 14B-720P layer as a
# conditional/unconditional pair, and a long 1080P-shaped sequence.
WORKLOADS = {
    0: Workload("tiny", 1, 2, 1024, 128, None, 64, 64, 0.25, True, False),
    1: Workload("wan1.3b-480p-dense", 1, 12, 32760, 128, (21, 30, 52), 128, 64, 1.0, False, False),
    2: Workload("wan1.3b-480p-sla", 1, 12, 32760, 128, (21, 30, 52), 128, 64, 0.10, True, True),
    3: Workload("wan14b-720p-sla-pair", 2, 40, 75600, 128, (21, 45, 80), 128, 64, 0.10, True, True),
    4: Workload("1080p-long-sla", 1, 40, 269280, 128, (33, 68, 120), 128, 64, 0.05, True, True),
}


def workload(i: int) -> Workload:
    return WORKLOADS[i]


def custom(B: int, H: int, N: int, *, D: int = 128, grid=None, blk_q: int = 128, blk_k: int = 64,
           topk_frac: float = 0.1, linear: bool = True, structured: bool = False, name: str = "custom") -> Workload:
    if structured:
        assert grid is not None and grid[0] * grid[1] * grid[2] == N, "structured inputs need a token grid"
    return Workload(name, B, H, N, D, grid, blk_q, blk_k, topk_frac, linear, structured)


_SIGMA = 2.0
_RADIUS = 8  # truncate at 4 sigma


def _blur_weights(device) -> torch.Tensor:
    i = torch.arange(-_RADIUS, _RADIUS + 1, dtype=torch.float64)
    w = torch.exp(-(i * i) / (2 * _SIGMA * _SIGMA))
    w = w / w.sum()
    return w.to(device=device, dtype=torch.float32)


def _mirror_index(L: int, device) -> torch.Tensor:
    # edge-including mirror: ... c b a | a b c ... | ... z y x | x y z ...
    # (repeated for axes shorter than the blur radius: the mirrored sequence has period 2L)
    idx = torch.remainder(torch.arange(-_RADIUS, L + _RADIUS, device=device), 2 * L)
    return torch.where(idx >= L, 2 * L - idx - 1, idx)


def _blur_axis(x: torch.Tensor, axis: int, w: torch.Tensor) -> torch.Tensor:
    x = x.movedim(axis, -1)
    shp = x.shape
    L = shp[-1]
    xp = x.reshape(-1, L).index_select(1, _mirror_index(L, x.device))
    y = torch.zeros_like(xp[:, :L])
    for i in range(2 * _RADIUS + 1):  # 17 shifted copies, weighted (no convolution library involved)
        y.add_(xp[:, i:i + L], alpha=float(w[i]))
    return y.reshape(shp).movedim(-1, axis)


def _smooth_field(noise: torch.Tensor) -> torch.Tensor:
    """noise [..., T, Hh, Ww] -> Gaussian-blurred field of the same shape, unit std over each grid."""
    w = _blur_weights(noise.device)
    f = noise
    for ax in (-3, -2, -1):
        f = _blur_axis(f, ax, w)
    return f / f.std(dim=(-3, -2, -1), keepdim=True)


@torch.no_grad()
def make(wl: Workload, seed: int = 0, device="cpu"):
    """Draw (q, k, v, w_p) for a workload: bf16 tensors, q/k/v [B, H, N, D] contiguous, w_p [D, D]."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    bias = 2.0 * torch.randn(H, D, generator=g, device=dev)
    w_p = torch.randn(D, D, generator=g, device=dev) / math.sqrt(D)
    q = torch.empty(B, H, N, D, dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    for b in range(B):
        if wl.structured:
            T, Hh, Ww = wl.grid
            noise = torch.randn(H, D, T, Hh, Ww, generator=g, device=dev)
            field = _smooth_field(noise).reshape(H, D, N).transpose(1, 2)  # [H, N, D]
            del noise
            qb = field + 0.3 * torch.randn(H, N, D, generator=g, device=dev)
            kb = field + 0.3 * torch.randn(H, N, D, generator=g, device=dev)
            del field
        else:
            qb = torch.randn(H, N, D, generator=g, device=dev)
            kb = torch.randn(H, N, D, generator=g, device=dev)
        vb = torch.randn(H, N, D, generator=g, device=dev)
        kb += bias[:, None, :]
        q[b].copy_(qb.to(torch.bfloat16))
        k[b].copy_(kb.to(torch.bfloat16))
        v[b].copy_(vb.to(torch.bfloat16))
        del qb, kb, vb
    return q, k, v, w_p.to(torch.bfloat16).contiguous()


# ---------------------------------------------------------------------------------------------------------
# W8A8 linear layers
# ---------------------------------------------------------------------------------------------------------
# The pages quantize the linear layers around attention with 8-bit weights and activations ("Turbo Diffusion",
# lanhy.cn, §三(四) item 1). Their shapes here are those of the Wan DiTs the pages accelerate: tokens M of one
# layer's input (the 14B 720P pair: 2 × 75600; the 1.3B 480P layer: 32760), model width 5120 (14B) or 1536
# (1.3B), FFN width 13824 (14B).
#
# Recipe (one torch.Generator seeded with ``seed``, in this order):
#   * chan[K]   = 1, except 1% of the input channels (chosen by a random permutation) set to 16: activation
#                 outlier channels, which make block absmax and clipping matter
#   * W[N, K]   = N(0,1) / sqrt(K)
#   * b[N]      = 0.1 N(0,1)
#   * X[M, K]   = N(0,1) * chan (drawn in row chunks to bound host memory)
#   * everything drawn in fp32 and rounded once to bf16.
@dataclasses.dataclass(frozen=True)
class LinearWorkload:
    name: str
    M: int  # tokens
    N: int  # output features
    K: int  # input features

    @property
    def ops(self) -> float:
        """2·M·N·K: multiply-adds of the product, counted as two operations each."""
        return 2.0 * self.M * self.N * self.K


LINEAR_WORKLOADS = {
    "small-ragged": LinearWorkload("small-ragged", 300, 384, 640),
    "wan1.3b-480p-proj": LinearWorkload("wan1.3b-480p-proj", 32760, 1536, 1536),
    "wan14b-720p-proj": LinearWorkload("wan14b-720p-proj", 151200, 5120, 5120),
    "wan14b-720p-ffn-up": LinearWorkload("wan14b-720p-ffn-up", 151200, 13824, 5120),
    "wan14b-720p-ffn-down": LinearWorkload("wan14b-720p-ffn-down", 151200, 5120, 13824),
    # the FFN-down layer at the most tokens the library takes for 13824 inputs (rows * cols < 2^31)
    "wan14b-ffn-down-max-rows": LinearWorkload("wan14b-ffn-down-max-rows", 155344, 5120, 13824),
}


def make_linear(wl: LinearWorkload, seed: int = 0, device="cpu", bias: bool = True):
    """Draw (x [M, K], w [N, K], b [N] or None): contiguous bf16 tensors."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    M, N, K = wl.M, wl.N, wl.K
    chan = torch.ones(K, device=dev)
    n_out = max(1, K // 100)
    chan[torch.randperm(K, generator=g, device=dev)[:n_out]] = 16.0
    w = (torch.randn(N, K, generator=g, device=dev) / math.sqrt(K)).to(torch.bfloat16)
    b = (0.1 * torch.randn(N, generator=g, device=dev)).to(torch.bfloat16)
    x = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    step = max(1, (1 << 26) // K)
    for r0 in range(0, M, step):
        r1 = min(M, r0 + step)
        x[r0:r1] = (torch.randn(r1 - r0, K, generator=g, device=dev) * chan).to(torch.bfloat16)
    return x, w, (b if bias else None)


# ---------------------------------------------------------------------------------------------------------
# RMSNorm weights of Q and K (the norm before the attention path)
# ---------------------------------------------------------------------------------------------------------
NORM_EPS = 1e-6  # the epsilon of the Wan DiTs' RMSNorm


def make_norm_weights(H: int, D: int, seed: int = 0, device="cpu"):
    """(gamma_q, gamma_k): bf16 [H*D] each, 1 + 0.1 N(0,1) drawn in fp32 from one generator seeded with
    ``seed`` (gamma_q first), rounded once to bf16."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed) + 7919)
    gq = (1.0 + 0.1 * torch.randn(H * D, generator=g, device=dev)).to(torch.bfloat16)
    gk = (1.0 + 0.1 * torch.randn(H * D, generator=g, device=dev)).to(torch.bfloat16)
    return gq, gk
