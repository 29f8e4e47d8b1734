"""Plain fp64 CPU oracle of the SLA backward for a fixed block selection.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this module: only the
tests use it. It shares no code with the HIP library; both sides only consume the same seeded inputs.

What is differentiated, and where the pages say so
--------------------------------------------------
[TD-news] ("Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破", lanhy.cn) calls SLA trainable: §三(二)
describes the sparse-plus-linear attention, and §四 step 1 fine-tunes the model with it before distillation.
The pages give no backward. Reading (the plainest one): the gradient of the float forward for a fixed
selection,
    F(Q, K, V, W_p) = O_s + O_l W_p
    O_s[i] = sum_j softmax_j(q_i . k_j * sm_scale) v_j over the keys j of the selected blocks of i's query block
    O_l[i] = phi(q_i) H_m / (phi(q_i) . Z_m), H_m, Z_m = sum over the unselected key blocks of phi(K_J)^T V_J and
             of the rows of phi(K_J); phi = elu + 1; O_l = 0 when every block is selected or linear is off,
with INT8 quantization passed straight through (the codes dequantize to the inputs) and K-mean smoothing
dropped (it shifts every score of a row by the same amount, so no softmax row, and no gradient, changes).
Given dY = dL/dF, the backward returns dQ, dK, dV of each head and dW_p summed over the heads (W_p is shared).

With the RMSNorm of Q and K before the path ([TD-news] §三(四) item 2 point 1), the reading is the same
straight-through one: the attention's gradient is taken at the normalized values the forward uses (Q-hat, K-hat
after their bf16 roundings, which pass gradients unchanged), then through the float RMSNorm
y_c = x_c r w_c (r = 1 / sqrt(mean over the token's H*D channels of x^2 + eps)) to the raw Q, K and the weights.

The gradient is computed by torch's reverse-mode differentiation (fp64, CPU) of that forward written out
plainly below, one query block at a time; the tests pin it against central finite differences of the same
forward and, for the dense special case, against torch's scaled_dot_product_attention.
"""
from __future__ import annotations

import math

import numpy as np
import torch

__all__ = ["forward_float_head", "backward_head", "backward", "dq_blocks", "rmsnorm_backward", "backward_with_norm"]


def _blocks(n, blk):
    return [(i * blk, min(n, (i + 1) * blk)) for i in range((n + blk - 1) // blk)]


def forward_float_head(Q, K, V, W_p, idx, blk_q, blk_k, sm_scale=None, linear=True):
    """F for one (b, h) head as fp64 torch tensors (differentiable); idx [n_qb][k] selected key blocks."""
    N, D = Q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    kblocks = _blocks(N, blk_k)
    phiQ = torch.where(Q > 0, Q + 1.0, torch.exp(torch.clamp(Q, max=0.0)))
    phiK = torch.where(K > 0, K + 1.0, torch.exp(torch.clamp(K, max=0.0)))
    rows_out = []
    for I, (r0, r1) in enumerate(_blocks(N, blk_q)):
        sel = sorted(set(int(J) for J in idx[I]))
        o = torch.zeros(r1 - r0, D, dtype=Q.dtype)
        if sel:
            keys = torch.cat([torch.arange(*kblocks[J]) for J in sel])
            p = torch.softmax((Q[r0:r1] @ K[keys].T) * sm_scale, dim=1)
            o = o + p @ V[keys]
        uns = [J for J in range(len(kblocks)) if J not in sel]
        if linear and uns:
            keys = torch.cat([torch.arange(*kblocks[J]) for J in uns])
            Hm = phiK[keys].T @ V[keys]
            Zm = phiK[keys].sum(dim=0)
            o = o + ((phiQ[r0:r1] @ Hm) / (phiQ[r0:r1] @ Zm)[:, None]) @ W_p
        rows_out.append(o)
    return torch.cat(rows_out, dim=0)


def backward_head(Q, K, V, W_p, idx, dY, blk_q, blk_k, sm_scale=None, linear=True):
    """dQ, dK, dV (fp64 [N, D]) and this head's dW_p ([D, D]) for one head; inputs are arrays of exact values."""
    t = lambda a: torch.tensor(np.asarray(a, np.float64), dtype=torch.float64, requires_grad=True)
    Qt, Kt, Vt, Wt = t(Q), t(K), t(V), t(W_p)
    F = forward_float_head(Qt, Kt, Vt, Wt, idx, blk_q, blk_k, sm_scale, linear)
    (F * torch.as_tensor(np.asarray(dY, np.float64))).sum().backward()
    return (Qt.grad.numpy(), Kt.grad.numpy(), Vt.grad.numpy(),
            (Wt.grad.numpy() if Wt.grad is not None else np.zeros_like(np.asarray(W_p, np.float64))))


def backward(q, k, v, w_p, idx, dy, blk_q, blk_k, sm_scale=None, linear=True, heads=None):
    """Batched: q, k, v, dy [B, H, N, D], idx [B, H, n_qb, k]. Returns (dq, dk, dv) dicts keyed by (b, h) for
    the requested heads (all by default) and dW_p summed over those heads."""
    B, H = np.asarray(q).shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    dq, dk, dv = {}, {}, {}
    dW = np.zeros_like(np.asarray(w_p, np.float64))
    for (b, h) in heads:
        gq, gk, gv, gw = backward_head(q[b][h], k[b][h], v[b][h], w_p, idx[b][h], dy[b][h], blk_q, blk_k,
                                       sm_scale, linear)
        dq[b, h], dk[b, h], dv[b, h] = gq, gk, gv
        dW += gw
    return dq, dk, dv, dW


def dq_blocks(Q, K, V, W_p, idx, dY, blk_q, blk_k, blocks, sm_scale=None, linear=True):
    """The rows of dQ for the query blocks `blocks` alone: the output of a query block depends on Q only through
    that block's own rows, so the gradient of the forward restricted to those blocks gives these rows exactly.
    Returns {I: dQ rows [rows of I, D]}."""
    N, D = np.asarray(Q).shape
    out = {}
    Kt = torch.as_tensor(np.asarray(K, np.float64))
    Vt = torch.as_tensor(np.asarray(V, np.float64))
    Wt = torch.as_tensor(np.asarray(W_p, np.float64))
    for I in blocks:
        r0, r1 = I * blk_q, min(N, (I + 1) * blk_q)
        Qb = torch.tensor(np.asarray(Q, np.float64)[r0:r1], requires_grad=True)
        # the block's rows as a query block of its own, against all keys (its selection unchanged)
        Qfull = torch.cat([torch.zeros(r0, D, dtype=torch.float64), Qb,
                           torch.zeros(N - r1, D, dtype=torch.float64)]) if (r0 or r1 < N) else Qb
        nq = (N + blk_q - 1) // blk_q
        sel = [idx[J] if J == I else [] for J in range(nq)]
        F = forward_float_head(Qfull, Kt, Vt, Wt, sel, blk_q, blk_k, sm_scale, linear=False)[r0:r1]
        if linear:
            F = F + _linear_rows(Qb, Kt, Vt, Wt, idx[I], blk_k)
        (F * torch.as_tensor(np.asarray(dY, np.float64)[r0:r1])).sum().backward()
        out[I] = Qb.grad.numpy()
    return out


def _linear_rows(Qb, K, V, W_p, sel, blk_k):
    """The linear branch of one query block's rows (phi(q) H_m / phi(q) . Z_m over its unselected key blocks)."""
    N = K.shape[0]
    kb = _blocks(N, blk_k)
    s = set(int(J) for J in sel)
    uns = [J for J in range(len(kb)) if J not in s]
    if not uns:
        return torch.zeros_like(Qb)
    keys = torch.cat([torch.arange(*kb[J]) for J in uns])
    phiK = torch.where(K[keys] > 0, K[keys] + 1.0, torch.exp(torch.clamp(K[keys], max=0.0)))
    phiQ = torch.where(Qb > 0, Qb + 1.0, torch.exp(torch.clamp(Qb, max=0.0)))
    Hm = phiK.T @ V[keys]
    Zm = phiK.sum(dim=0)
    return ((phiQ @ Hm) / (phiQ @ Zm)[:, None]) @ W_p


def rmsnorm_backward(X, gamma, eps, dY):
    """Backward of the RMSNorm before the path for one batch entry (straight-through roundings): X [H, N, D] raw
    values, gamma [H*D] (index h*D + d), dY [H, N, D] = dL/d(normalized). Per token, with c over its n = H*D
    channels and r = 1 / sqrt(sum_c x_c^2 / n + eps):
        dL/dx_c = r w_c dy_c - x_c r^3 / n * sum_c' x_c' w_c' dy_c'
        dL/dw_c = sum over the tokens of x_c r dy_c
    (fp64). Returns (dX [H, N, D], dgamma [H*D])."""
    X = np.asarray(X, np.float64)
    H, N, D = X.shape
    x = X.transpose(1, 0, 2).reshape(N, H * D)                 # token-major rows of n channels
    dy = np.asarray(dY, np.float64).transpose(1, 0, 2).reshape(N, H * D)
    w = np.asarray(gamma, np.float64).reshape(1, H * D)
    n = float(H * D)
    r = 1.0 / np.sqrt((x * x).sum(axis=1, keepdims=True) / n + float(np.float32(eps)))
    s_ = (x * w * dy).sum(axis=1, keepdims=True)
    dx = r * w * dy - x * (r ** 3) / n * s_
    dw = (x * r * dy).sum(axis=0)
    return dx.reshape(N, H, D).transpose(1, 0, 2), dw


def backward_with_norm(q, k, v, w_p, idx, dy, blk_q, blk_k, gq, gk, eps, sm_scale=None, linear=True):
    """The whole backward with the RMSNorm of Q and K before the path: q, k, v, dy [B, H, N, D] raw values,
    gq, gk [H*D]. The attention part runs at the forward's normalized values (the oracle's qk_rmsnorm, the same
    bf16 values the forward computes) and its dQ-hat, dK-hat pass through rmsnorm_backward. Returns (dq, dk, dv
    as [B, H, N, D] arrays, dW_p, dgq, dgk), the weight gradients summed over the batch entries."""
    from oracle.sagesla import qk_rmsnorm
    q, k, v, dy = (np.asarray(a, np.float64) for a in (q, k, v, dy))
    B, H, N, D = q.shape
    qh = np.stack([qk_rmsnorm(q[b], gq, eps)[0] for b in range(B)])
    kh = np.stack([qk_rmsnorm(k[b], gk, eps)[0] for b in range(B)])
    dqh, dkh, dvd, dW = backward(qh, kh, v, w_p, idx, dy, blk_q, blk_k, sm_scale, linear)
    dq, dk = np.zeros_like(q), np.zeros_like(k)
    dv = np.zeros_like(v)
    dgq, dgk = np.zeros(H * D), np.zeros(H * D)
    for b in range(B):
        gqh = np.stack([dqh[b, h] for h in range(H)])
        gkh = np.stack([dkh[b, h] for h in range(H)])
        dq[b], wq_ = rmsnorm_backward(q[b], gq, eps, gqh)
        dk[b], wk_ = rmsnorm_backward(k[b], gk, eps, gkh)
        dgq += wq_
        dgk += wk_
        for h in range(H):
            dv[b, h] = dvd[b, h]
    return dq, dk, dv, dW, dgq, dgk
