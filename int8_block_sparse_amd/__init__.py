"""SageSLA attention forward for AMD Instinct MI355X (gfx950): thin Python binding of libsagesla.so.

Every step of the forward runs in the library's HIP kernels; this module only marshals arguments through the
C ABI declared in include/sagesla.h (the W8A8 linear layer of include/w8a8.h is bound in w8a8.py). PyTorch provides device memory and the current stream. There is no CPU
fallback: calls fail loudly if the library is missing or no GPU is present.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

__all__ = [
    "LIB_PATH", "load", "Params", "SageSLAError", "topk_blocks", "n_blocks", "workspace_bytes", "validate",
    "quantize", "select", "forward", "LINEAR", "SMOOTH_K", "USE_GIVEN_MASK", "QUANT_GROUP32", "QK_RMSNORM", "STATUS", "STAGES",
    "stage_events",
    "stage_ms", "Config", "backward", "forward_noalloc", "NOALLOC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsagesla.so")

LINEAR = 0x1
SMOOTH_K = 0x2
USE_GIVEN_MASK = 0x4
QUANT_GROUP32 = 0x8  # one INT8 scale per 32 tokens of Q and of K (thread-level granularity)
QK_RMSNORM = 0x10  # RMSNorm of Q and K over all heads of each token first

NOALLOC_SCRATCH_BYTES = 64 << 20  # SAGESLA_NOALLOC_SCRATCH_BYTES
STATUS = {0: "OK", 1: "E_NULL", 2: "E_SHAPE", 3: "E_UNSUPPORTED", 4: "E_WORKSPACE", 5: "E_ALIGN", 6: "E_HIP"}
STAGES = ("quantize", "select", "linear", "attn")


class SageSLAError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({_lib_status_str(status)})"
        if status == 6:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


class Params(ctypes.Structure):
    """Mirror of struct sagesla_params."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32),
        ("blk_q", ctypes.c_int32), ("blk_k", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("sm_scale", ctypes.c_float),
        ("w_proj", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("q_i8", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("k_i8", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("k_mean", ctypes.c_void_p), ("q_pool", ctypes.c_void_p),
        ("k_pool", ctypes.c_void_p), ("block_idx", ctypes.c_void_p), ("o_lin", ctypes.c_void_p),
        ("events", ctypes.POINTER(ctypes.c_void_p)),
        ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p), ("q_hat", ctypes.c_void_p),
        ("k_hat", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
        ("dq_norm_w", ctypes.c_void_p), ("dk_norm_w", ctypes.c_void_p), ("scores", ctypes.c_void_p),
    ]


_lib = None


def load():
    """Load libsagesla.so (built by __graft_entry__.build() / python -m int8_block_sparse_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m int8_block_sparse_amd.build`")
    # torch first: the library's HIP runtime dependency then binds to the runtime torch already loaded, so
    # torch's device memory, streams and events are the library's too
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Params)
    vp = ctypes.c_void_p
    lib.sagesla_workspace_bytes.argtypes = [P]
    lib.sagesla_workspace_bytes.restype = ctypes.c_size_t
    lib.sagesla_validate.argtypes = [P]
    lib.sagesla_validate.restype = ctypes.c_int
    lib.sagesla_quantize.argtypes = [vp, vp, P, vp]
    lib.sagesla_quantize.restype = ctypes.c_int
    lib.sagesla_select.argtypes = [P, vp]
    lib.sagesla_select.restype = ctypes.c_int
    lib.sagesla_forward.argtypes = [vp, vp, vp, vp, P, vp]
    lib.sagesla_forward.restype = ctypes.c_int
    lib.sagesla_forward_noalloc.argtypes = [vp, vp, vp, vp, P, vp]
    lib.sagesla_forward_noalloc.restype = ctypes.c_int
    lib.sagesla_backward_workspace_bytes.argtypes = [P]
    lib.sagesla_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.sagesla_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, P, vp]
    lib.sagesla_backward.restype = ctypes.c_int
    lib.sagesla_status_str.argtypes = [ctypes.c_int]
    lib.sagesla_status_str.restype = ctypes.c_char_p
    lib.sagesla_last_hip_error.argtypes = []
    lib.sagesla_last_hip_error.restype = ctypes.c_int
    i32, f32 = ctypes.c_int32, ctypes.c_float
    lib.w8a8_quantize.argtypes = [vp, i32, i32, f32, vp, vp, vp]
    lib.w8a8_quantize.restype = ctypes.c_int
    lib.w8a8_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.w8a8_gemm.restype = ctypes.c_int
    lib.w8a8_workspace_bytes.argtypes = [i32, i32]
    lib.w8a8_workspace_bytes.restype = ctypes.c_size_t
    lib.w8a8_linear.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32, vp, ctypes.c_size_t, vp]
    lib.w8a8_linear.restype = ctypes.c_int
    _lib = lib
    return lib


def _lib_status_str(status: int) -> str:
    try:
        return load().sagesla_status_str(status).decode()
    except Exception:  # noqa: BLE001 - message helper only
        return "?"


def n_blocks(n: int, blk: int) -> int:
    return -(-n // blk)


def topk_blocks(frac: float, n_kb: int) -> int:
    """Key blocks kept per query block for the --sla_topk fraction: round half up, at least 1, all for frac >= 1."""
    if frac >= 1.0:
        return n_kb
    return max(1, int(math.floor(frac * n_kb + 0.5)))


@dataclass
class Config:
    B: int
    H: int
    N: int
    D: int = 128
    blk_q: int = 128
    blk_k: int = 64
    topk: int = 0
    linear: bool = True
    smooth_k: bool = True
    sm_scale: float = 0.0
    group32: bool = False  # one INT8 scale per 32 tokens instead of one per block
    qk_norm: bool = False  # RMSNorm of Q and K first (weights and eps passed as pointers / norm_eps)

    @property
    def n_qb(self) -> int:
        return n_blocks(self.N, self.blk_q)

    @property
    def n_kb(self) -> int:
        return n_blocks(self.N, self.blk_k)

    @property
    def n_qscale(self) -> int:
        return n_blocks(self.N, 32) if self.group32 else self.n_qb

    @property
    def n_kscale(self) -> int:
        return n_blocks(self.N, 32) if self.group32 else self.n_kb

    def params(self, **ptrs) -> Params:
        flags = ((LINEAR if self.linear else 0) | (SMOOTH_K if self.smooth_k else 0) |
                 (QUANT_GROUP32 if self.group32 else 0) | (QK_RMSNORM if self.qk_norm else 0))
        if ptrs.pop("given_mask", False):
            flags |= USE_GIVEN_MASK
        p = Params(B=self.B, H=self.H, N=self.N, D=self.D, blk_q=self.blk_q, blk_k=self.blk_k, topk=self.topk,
                   flags=flags, sm_scale=self.sm_scale)
        for k, v in ptrs.items():
            setattr(p, k, v)
        return p


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise SageSLAError(status, where, load().sagesla_last_hip_error())


def validate(cfg: Config) -> int:
    return load().sagesla_validate(ctypes.byref(cfg.params()))


def workspace_bytes(cfg: Config) -> int:
    n = load().sagesla_workspace_bytes(ctypes.byref(cfg.params()))
    if n == 0:
        _check(validate(cfg) or 2, "sagesla_workspace_bytes")
    return n


def _workspace(cfg: Config, device, workspace):
    import torch
    need = workspace_bytes(cfg)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def _shape_check(q, k, v, out, cfg: Config):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t is None:
            continue
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
        if tuple(t.shape) != (cfg.B, cfg.H, cfg.N, cfg.D):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(cfg.B, cfg.H, cfg.N, cfg.D)}")


def _exports(cfg: Config, device):
    import torch
    BH, N, D = cfg.B * cfg.H, cfg.N, cfg.D
    f = dict(device=device)
    ex = {
        "q_i8": torch.empty(cfg.B, cfg.H, N, D, dtype=torch.int8, **f),
        "q_scale": torch.empty(cfg.B, cfg.H, cfg.n_qscale, dtype=torch.float32, **f),
        "k_i8": torch.empty(cfg.B, cfg.H, N, D, dtype=torch.int8, **f),
        "k_scale": torch.empty(cfg.B, cfg.H, cfg.n_kscale, dtype=torch.float32, **f),
        "k_mean": torch.empty(cfg.B, cfg.H, D, dtype=torch.float32, **f),
        "q_pool": torch.empty(cfg.B, cfg.H, cfg.n_qb, D, dtype=torch.float64, **f),
        "k_pool": torch.empty(cfg.B, cfg.H, cfg.n_kb, D, dtype=torch.float64, **f),
        "block_idx": torch.empty(cfg.B, cfg.H, cfg.n_qb, max(cfg.topk, 1), dtype=torch.int32, **f),
    }
    if 0 < cfg.topk < cfg.n_kb:  # the block scores the top-k ranks (written when the selection runs)
        ex["scores"] = torch.empty(cfg.B, cfg.H, cfg.n_qb, cfg.n_kb, dtype=torch.float64, **f)
    if cfg.linear:
        ex["o_lin"] = torch.empty(cfg.B, cfg.H, N, D, dtype=torch.float32, **f)
    if cfg.qk_norm:
        ex["q_hat"] = torch.empty(cfg.B, cfg.H, N, D, dtype=torch.bfloat16, **f)
        ex["k_hat"] = torch.empty(cfg.B, cfg.H, N, D, dtype=torch.bfloat16, **f)
    del BH
    return ex


def stage_events():
    """2 * len(STAGES) timing events for forward(events=...); read them with stage_ms() after synchronizing."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(STAGES))]
    for e in evs:
        e.record()  # creates the underlying hipEvent_t
    return evs


def stage_ms(evs):
    """Per-stage milliseconds from events recorded by forward(events=evs)."""
    return {name: evs[2 * i].elapsed_time(evs[2 * i + 1]) for i, name in enumerate(STAGES)}


def _norm_args(norm, H, D):
    """(gamma_q, gamma_k, eps) -> Params fields; gammas bf16 [H*D] CUDA tensors."""
    import torch
    if norm is None:
        return {}
    gq, gk, eps = norm
    for name, t in (("gamma_q", gq), ("gamma_k", gk)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.numel() != H * D:
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor of H*D elements")
    return {"q_norm_w": gq.data_ptr(), "k_norm_w": gk.data_ptr(), "norm_eps": float(eps)}


def forward(q, k, v, w_proj=None, *, topk: int, blk_q: int = 128, blk_k: int = 64, linear: bool = True,
            smooth_k: bool = True, sm_scale: float = 0.0, mask=None, out=None, workspace=None,
            export: bool = False, events=None, group32: bool = False, norm=None):
    """SageSLA forward. q, k, v: bf16 [B, H, N, 128] CUDA tensors; w_proj: bf16 [128, 128] (needed with linear).

    mask: optional int32 [B, H, n_qb, topk] ascending block lists used instead of the selection.
    group32: one INT8 scale per 32 tokens of Q and of K instead of one per block.
    norm: (gamma_q, gamma_k, eps) normalizes Q and K first (RMSNorm over the H*D channels of each token).
    export=True also returns a dict of every intermediate (codes, scales, K mean, pooled means, block scores when
    the selection runs, block lists, and the linear-branch output). Runs asynchronously on the current stream."""
    return _forward(q, k, v, w_proj, topk, blk_q, blk_k, linear, smooth_k, sm_scale, mask, out, workspace, export,
                    events, group32, norm, noalloc=False)


def forward_noalloc(q, k, v, w_proj=None, *, topk: int, blk_q: int = 128, blk_k: int = 64, linear: bool = True,
                    smooth_k: bool = True, sm_scale: float = 0.0, mask=None, out=None, export: bool = False,
                    events=None, group32: bool = False, norm=None):
    """forward() through sagesla_forward_noalloc: no workspace argument; the library's own device scratch of
    NOALLOC_SCRATCH_BYTES serves (calls that overlap on one GPU race). Same results as forward()."""
    return _forward(q, k, v, w_proj, topk, blk_q, blk_k, linear, smooth_k, sm_scale, mask, out, None, export,
                    events, group32, norm, noalloc=True)


def _forward(q, k, v, w_proj, topk, blk_q, blk_k, linear, smooth_k, sm_scale, mask, out, workspace, export, events,
             group32, norm, noalloc):
    B, H, N, D = q.shape
    cfg = Config(B, H, N, D, blk_q, blk_k, topk, linear, smooth_k, sm_scale, group32, norm is not None)
    if out is None:
        import torch
        out = torch.empty_like(q)
    _shape_check(q, k, v, out, cfg)
    ws = None if noalloc else _workspace(cfg, q.device, workspace)
    ex = _exports(cfg, q.device) if export else {}
    if mask is not None:
        if not export:
            ex = {}
        ex["block_idx"] = mask
        ex.pop("scores", None)  # a given mask skips the selection
    ptrs = {name: _ptr(t) for name, t in ex.items()}
    p = cfg.params(w_proj=_ptr(w_proj), workspace=None if noalloc else ws.data_ptr(),
                   workspace_bytes=0 if noalloc else ws.numel(), given_mask=mask is not None, **ptrs,
                   **_norm_args(norm, H, D))
    if events is not None:
        arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        p.events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    fn = load().sagesla_forward_noalloc if noalloc else load().sagesla_forward
    _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), ctypes.byref(p), _stream(q.device)),
           "sagesla_forward_noalloc" if noalloc else "sagesla_forward")
    return (out, ex) if export else out


def quantize(q, k, *, blk_q: int = 128, blk_k: int = 64, smooth_k: bool = True, workspace=None,
             group32: bool = False, norm=None):
    """Quantize stage alone: returns dict(q_i8, q_scale, k_i8, k_scale, k_mean, q_pool, k_pool) and the workspace
    (pass it to select())."""
    B, H, N, D = q.shape
    cfg = Config(B, H, N, D, blk_q, blk_k, 0, False, smooth_k, group32=group32, qk_norm=norm is not None)
    _shape_check(q, k, None, None, cfg)
    ws = _workspace(cfg, q.device, workspace)
    ex = _exports(cfg, q.device)
    ex.pop("block_idx")
    p = cfg.params(workspace=ws.data_ptr(), workspace_bytes=ws.numel(), **{n: _ptr(t) for n, t in ex.items()},
                   **_norm_args(norm, H, D))
    _check(load().sagesla_quantize(q.data_ptr(), k.data_ptr(), ctypes.byref(p), _stream(q.device)),
           "sagesla_quantize")
    return ex, ws


def select(q_pool, k_pool, *, N: int, topk: int, blk_q: int = 128, blk_k: int = 64, workspace=None):
    """Select stage alone from pooled means (fp64 [B, H, n_blocks, 128]); returns int32 [B, H, n_qb, topk]."""
    import torch
    B, H = q_pool.shape[:2]
    cfg = Config(B, H, N, q_pool.shape[-1], blk_q, blk_k, topk, False, True)
    ws = _workspace(cfg, q_pool.device, workspace)
    idx = torch.empty(B, H, cfg.n_qb, max(topk, 1), dtype=torch.int32, device=q_pool.device)
    qp, kp = q_pool.contiguous(), k_pool.contiguous()
    p = cfg.params(workspace=ws.data_ptr(), workspace_bytes=ws.numel(), q_pool=qp.data_ptr(),
                   k_pool=kp.data_ptr(), block_idx=idx.data_ptr())
    _check(load().sagesla_select(ctypes.byref(p), _stream(q_pool.device)), "sagesla_select")
    return idx[..., :topk]


def backward(q, k, v, w_proj, dout, mask, *, topk: int, blk_q: int = 128, blk_k: int = 64, linear: bool = True,
             sm_scale: float = 0.0, workspace=None, norm=None):
    """SLA backward for the fixed selection `mask` (int32 [B, H, n_qb, topk]): gradient of the float forward
    (INT8 quantization straight through) given dout = dL/d(out) (bf16 [B, H, N, 128]). Returns fp32 (dq, dk, dv)
    and dW_p (fp32 [128, 128], summed over every head; None without the linear branch). With norm =
    (gamma_q, gamma_k, eps), the RMSNorm of Q and K before the path (as in forward): dq, dk are the gradients of the
    raw q, k, and the norm weights' gradients (fp32 [H*128] each) follow dW_p in the result. Runs on the current
    stream."""
    import torch
    B, H, N, D = q.shape
    cfg = Config(B, H, N, D, blk_q, blk_k, topk, linear, True, sm_scale, False, norm is not None)
    _shape_check(q, k, v, dout, cfg)
    if topk > 0 and (mask is None or mask.dtype != torch.int32 or not mask.is_contiguous()
                     or tuple(mask.shape) != (B, H, cfg.n_qb, topk)):
        raise ValueError("mask must be a contiguous int32 CUDA tensor [B, H, n_qb, topk]")
    nargs = _norm_args(norm, H, D)
    p0 = cfg.params(w_proj=_ptr(w_proj), **nargs)
    need = load().sagesla_backward_workspace_bytes(ctypes.byref(p0))
    if need == 0:
        _check(validate(cfg) or 3, "sagesla_backward_workspace_bytes")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq, dk, dv = (torch.empty(B, H, N, D, **f32) for _ in range(3))
    dw = torch.empty(D, D, **f32) if linear else None
    dwn = (torch.empty(H * D, **f32), torch.empty(H * D, **f32)) if norm is not None else (None, None)
    p = cfg.params(w_proj=_ptr(w_proj), workspace=workspace.data_ptr(), workspace_bytes=workspace.numel(),
                   block_idx=_ptr(mask) if topk > 0 else None, dq_norm_w=_ptr(dwn[0]), dk_norm_w=_ptr(dwn[1]),
                   **nargs)
    _check(load().sagesla_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                   dk.data_ptr(), dv.data_ptr(), _ptr(dw), ctypes.byref(p), _stream(q.device)),
           "sagesla_backward")
    return (dq, dk, dv, dw) if norm is None else (dq, dk, dv, dw, dwn[0], dwn[1])
