"""Pins of the SLA-backward oracle (CPU only): central finite differences of the float forward in every input
direction class, and the dense special case against torch's scaled_dot_product_attention backward."""
import math

import numpy as np
import pytest
import torch

from oracle import sla_backward as ob
from oracle import sagesla as orc


def _case(N=200, D=128, blk_q=64, blk_k=64, k=2, seed=0):
    rng = np.random.default_rng(seed)
    Q, K, V = (orc.bf16_round(rng.standard_normal((N, D))) for _ in range(3))
    K = orc.bf16_round(K + rng.standard_normal(D))  # a channel bias, as the forward's inputs carry
    W = orc.bf16_round(rng.standard_normal((D, D)) / math.sqrt(D))
    nqb, nkb = -(-N // blk_q), -(-N // blk_k)
    idx = np.stack([np.sort(rng.choice(nkb, k, replace=False)) for _ in range(nqb)]).astype(np.int32)
    dY = rng.standard_normal((N, D))
    return Q, K, V, W, idx, dY


def _loss(Q, K, V, W, idx, dY, blk_q, blk_k, linear):
    T = lambda a: torch.as_tensor(np.asarray(a, np.float64))
    F = ob.forward_float_head(T(Q), T(K), T(V), T(W), idx, blk_q, blk_k, linear=linear)
    return float((F * T(dY)).sum())


@pytest.mark.parametrize("k,linear", [(2, True), (1, False), (0, True), (4, True)], ids=["mixed", "sparse",
                                                                                          "linear", "all"])
def test_finite_differences(k, linear):
    Q, K, V, W, idx, dY = _case(k=k)
    idx = idx[:, :k] if k else np.zeros((idx.shape[0], 0), np.int32)
    gQ, gK, gV, gW = ob.backward_head(Q, K, V, W, idx, dY, 64, 64, linear=linear)
    rng = np.random.default_rng(1)
    eps = 1e-5
    for name, x, g in (("Q", Q, gQ), ("K", K, gK), ("V", V, gV), ("W", W, gW)):
        d = rng.standard_normal(x.shape)
        args = {"Q": Q, "K": K, "V": V, "W": W}
        lp = dict(args, **{name: x + eps * d})
        lm = dict(args, **{name: x - eps * d})
        fd = (_loss(lp["Q"], lp["K"], lp["V"], lp["W"], idx, dY, 64, 64, linear) -
              _loss(lm["Q"], lm["K"], lm["V"], lm["W"], idx, dY, 64, 64, linear)) / (2 * eps)
        an = float(np.sum(g * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"d{name}: finite difference {fd} vs {an}"
    if not linear:
        assert not gW.any()


def test_dense_matches_library_attention_backward():
    Q, K, V, W, idx, dY = _case(N=192, k=3)
    idx = np.tile(np.arange(3, dtype=np.int32), (3, 1))
    gQ, gK, gV, _ = ob.backward_head(Q, K, V, W, idx, dY, 64, 64, linear=False)
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    q, k, v = t(Q), t(K), t(V)
    o = torch.nn.functional.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None],
                                                         scale=1 / math.sqrt(128))[0, 0]
    (o * torch.as_tensor(dY)).sum().backward()
    for a, b in ((gQ, q.grad), (gK, k.grad), (gV, v.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)


def test_forward_float_matches_quantization_free_forward():
    # the differentiated forward is the forward oracle's own unquantized, unsmoothed path on the same selection
    # (smoothing would only add the fp32 rounding of K - mu)
    Q, K, V, W, idx, dY = _case(N=300, k=2)
    F = ob.forward_float_head(*(torch.as_tensor(a) for a in (Q, K, V, W)), idx, 64, 64).numpy()
    r = orc.forward_head(Q, K, V, W, 64, 64, 2, quant=False, smooth_k=False, mask=idx)
    np.testing.assert_allclose(F, r["out"], rtol=1e-9, atol=1e-10)


def _fwd_no_scale(Q, K, V, W_p, idx, blk_q, blk_k, sm_scale=None, linear=True):
    return _orig_fwd(Q, K, V, W_p, idx, blk_q, blk_k, 1.0, linear)


def _fwd_linear_over_selected(Q, K, V, W_p, idx, blk_q, blk_k, sm_scale=None, linear=True):
    nkb = -(-K.shape[0] // blk_k)
    comp = [[J for J in range(nkb) if J not in set(int(x) for x in row)] for row in idx]
    sparse = _orig_fwd(Q, K, V, W_p, idx, blk_q, blk_k, sm_scale, linear=False)
    full = _orig_fwd(Q, K, V, W_p, comp, blk_q, blk_k, sm_scale, linear=linear)
    nolin = _orig_fwd(Q, K, V, W_p, comp, blk_q, blk_k, sm_scale, linear=False)
    return sparse + (full - nolin)  # the linear part taken over the selected blocks instead


_orig_fwd = ob.forward_float_head


@pytest.mark.parametrize("mut", [_fwd_no_scale, _fwd_linear_over_selected], ids=["no_scale", "linear_selected"])
def test_planted_forward_mistakes_are_caught(mut, monkeypatch):
    monkeypatch.setattr(ob, "forward_float_head", mut)
    with pytest.raises(AssertionError):
        test_forward_float_matches_quantization_free_forward()


def test_dq_blocks_equals_full_backward():
    Q, K, V, W, idx, dY = _case(N=330, k=2)
    gQ, _, _, _ = ob.backward_head(Q, K, V, W, idx, dY, 64, 64)
    part = ob.dq_blocks(Q, K, V, W, idx, dY, 64, 64, [0, 2, 5])
    for I, rows in part.items():
        np.testing.assert_allclose(rows, gQ[I * 64:min(330, I * 64 + 64)], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------------------------------------
# the RMSNorm before the path: its backward pinned to torch's own rms_norm differentiated in fp64, and the
# whole chain to central finite differences of the float forward through the float norm
# ---------------------------------------------------------------------------------------------------------
def test_rmsnorm_backward_matches_library_autograd():
    import torch.nn.functional as F
    rng = np.random.default_rng(5)
    H, N, D = 3, 7, 128
    X = rng.standard_normal((H, N, D)) * rng.uniform(0.2, 3.0, size=(1, N, 1))
    g = 1.0 + 0.1 * rng.standard_normal(H * D)
    dY = rng.standard_normal((H, N, D))
    eps = 1e-6
    dX, dg = ob.rmsnorm_backward(X, g, eps, dY)
    x = torch.tensor(X.transpose(1, 0, 2).reshape(N, H * D), dtype=torch.float64, requires_grad=True)
    w = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    y = F.rms_norm(x, (H * D,), weight=w, eps=float(np.float32(eps)))
    (y * torch.tensor(dY.transpose(1, 0, 2).reshape(N, H * D))).sum().backward()
    np.testing.assert_allclose(dX, x.grad.numpy().reshape(N, H, D).transpose(1, 0, 2), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dg, w.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_backward_with_norm_finite_differences():
    # a float chain without roundings: the oracle's norm step is replaced by the float norm, so the straight-
    # through gradient equals the exact derivative of the composed float function
    import oracle.sagesla as osg
    from types import SimpleNamespace
    wl = SimpleNamespace(H=2, N=150, D=128, blk_q=64, blk_k=64)
    wl.n_qb, wl.n_kb = (wl.N + 63) // 64, (wl.N + 63) // 64
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, wl.H, wl.N, wl.D)) for _ in range(3))
    w = rng.standard_normal((wl.D, wl.D)) / math.sqrt(wl.D)
    gq = 1.0 + 0.1 * rng.standard_normal(wl.H * wl.D)
    gk = 1.0 + 0.1 * rng.standard_normal(wl.H * wl.D)
    dy = rng.standard_normal(q.shape)
    idx = [[rng.choice(wl.n_kb, 1, replace=False) for _ in range(wl.n_qb)] for _ in range(wl.H)]
    idx = np.array(idx).reshape(1, wl.H, wl.n_qb, 1).astype(np.int32)
    eps = 1e-6

    def float_norm(X, gamma, eps_):
        X = np.asarray(X, np.float64)
        H, N, D = X.shape
        x = X.transpose(1, 0, 2).reshape(N, H * D)
        r = 1.0 / np.sqrt((x * x).sum(axis=1, keepdims=True) / (H * D) + float(np.float32(eps_)))
        return (x * r * np.asarray(gamma).reshape(1, -1)).reshape(N, H, D).transpose(1, 0, 2), None, None

    orig = osg.qk_rmsnorm
    osg.qk_rmsnorm = float_norm
    try:
        dq, dk, dv, dW, dgq, dgk = ob.backward_with_norm(q, k, v, w, idx, dy, wl.blk_q, wl.blk_k, gq, gk, eps)

        def L(qq, kk, ggq, ggk):
            qh = float_norm(qq[0], ggq, eps)[0]
            kh = float_norm(kk[0], ggk, eps)[0]
            tot = 0.0
            for h in range(wl.H):
                F_ = ob.forward_float_head(torch.tensor(qh[h]), torch.tensor(kh[h]), torch.tensor(v[0, h]),
                                           torch.tensor(np.asarray(w, np.float64)), idx[0, h], wl.blk_q, wl.blk_k)
                tot += float((F_.numpy() * dy[0, h]).sum())
            return tot

        rng2 = np.random.default_rng(7)
        for name, arr, grad in (("q", q, dq), ("k", k, dk)):
            for _ in range(3):
                h, n, d = rng2.integers(wl.H), rng2.integers(wl.N), rng2.integers(wl.D)
                e = 1e-5 * max(1.0, abs(arr[0, h, n, d]))
                ap, am = arr.copy(), arr.copy()
                ap[0, h, n, d] += e
                am[0, h, n, d] -= e
                fd = (L(ap, k, gq, gk) - L(am, k, gq, gk)) / (2 * e) if name == "q" else \
                     (L(q, ap, gq, gk) - L(q, am, gq, gk)) / (2 * e)
                assert abs(fd - grad[0, h, n, d]) <= 1e-6 * max(1.0, abs(fd)), (name, fd, grad[0, h, n, d])
        for name, gam, grad in (("gq", gq, dgq), ("gk", gk, dgk)):
            c = rng2.integers(wl.H * wl.D)
            e = 1e-5
            gp, gm = gam.copy(), gam.copy()
            gp[c] += e
            gm[c] -= e
            fd = (L(q, k, gp, gk) - L(q, k, gm, gk)) / (2 * e) if name == "gq" else \
                 (L(q, k, gq, gp) - L(q, k, gq, gm)) / (2 * e)
            assert abs(fd - grad[c]) <= 1e-6 * max(1.0, abs(fd)), (name, fd, grad[c])
    finally:
        osg.qk_rmsnorm = orig
