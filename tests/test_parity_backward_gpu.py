"""GPU parity of the SLA backward (sagesla_backward) with the fp64 oracle (oracle/sla_backward.py) on seeded
inputs and seeded selections.

Bar: for each of dQ, dK, dV (per head) and dW_p, relative L2 error <= 1e-4 and max-abs error <= 1e-3 of the
tensor's largest magnitude. The kernels form scores from exact bf16 inputs in fp32, the probabilities and dS
enter their products as bf16 hi + lo pairs (~2^-17 relative) and the linear branch starts from the forward's
remaining state in the same hi + lo form, so the expected relative error is ~1e-5.
"""
import numpy as np
import pytest
import torch

import int8_block_sparse_amd as sg
import synth
from conftest import to_np
from oracle import sla_backward as ob

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4
MAX_REL = 1e-3


def say(*a):
    print(*a, flush=True)


def close(name, got, want):
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    mx = np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-300)
    say(f"    {name}: rel-L2 {rel:.2e}, max-abs/max {mx:.2e}")
    assert rel <= REL_L2 and mx <= MAX_REL, f"{name}: rel-L2 {rel:.3e} max {mx:.3e}"


def make_mask(wl, topk, seed, dup=False):
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(wl.B * wl.H * wl.n_qb):
        r = np.sort(rng.choice(wl.n_kb, topk, replace=False)) if topk else np.zeros(0, np.int64)
        if dup and topk >= 2:
            r[-1] = r[0]  # a block listed twice counts once
        rows.append(r)
    return np.stack(rows).reshape(wl.B, wl.H, wl.n_qb, topk).astype(np.int32)


def case(wl, topk, linear=True, seed=0, dup=False):
    q, k, v, w = synth.make(wl, seed)
    dy = (torch.randn(q.shape, generator=torch.Generator().manual_seed(seed + 11))).to(torch.bfloat16)
    mask = make_mask(wl, topk, seed, dup)
    say(f"case {wl.name} B{wl.B} H{wl.H} N{wl.N} bq{wl.blk_q} topk{topk} linear{linear} dup{dup}")
    dq, dk, dv, dw = sg.backward(q.cuda(), k.cuda(), v.cuda(), w.cuda(), dy.cuda(), torch.from_numpy(mask).cuda(),
                                 topk=topk, blk_q=wl.blk_q, blk_k=wl.blk_k, linear=linear)
    torch.cuda.synchronize()
    rq, rk, rv, rw = ob.backward(to_np(q), to_np(k), to_np(v), to_np(w), mask, to_np(dy), wl.blk_q, wl.blk_k,
                                 linear=linear)
    for b in range(wl.B):
        for h in range(wl.H):
            say(f"  b{b} h{h}")
            close("dq", to_np(dq[b, h]), rq[b, h])
            close("dk", to_np(dk[b, h]), rk[b, h])
            close("dv", to_np(dv[b, h]), rv[b, h])
    if linear:
        if np.abs(rw).max() == 0:
            assert not to_np(dw).any()
        else:
            close("dW_p", to_np(dw), rw)


SMALL = {
    "ragged128": synth.custom(1, 2, 1000, blk_q=128, topk_frac=0.2),
    "ragged64": synth.custom(2, 1, 330, blk_q=64, topk_frac=0.34),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_backward_mixed(name):
    wl = SMALL[name]
    case(wl, max(1, wl.n_kb // 4))


def test_backward_sparse_only():
    case(SMALL["ragged128"], 3, linear=False)


def test_backward_linear_only():
    case(SMALL["ragged128"], 0)


def test_backward_all_selected():
    wl = SMALL["ragged64"]
    case(wl, wl.n_kb)


def test_backward_repeated_blocks():
    case(SMALL["ragged128"], 4, dup=True)


def test_backward_deterministic():
    wl = SMALL["ragged128"]
    q, k, v, w = (t.cuda() for t in synth.make(wl, 5))
    dy = torch.randn(q.shape, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()
    mask = torch.from_numpy(make_mask(wl, 3, 5)).cuda()
    a = sg.backward(q, k, v, w, dy, mask, topk=3)
    b = sg.backward(q, k, v, w, dy, mask, topk=3)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---------------------------------------------------------------------------------------------------------
# degenerate shapes and inputs
# ---------------------------------------------------------------------------------------------------------
def run(wl, topk, seed=0, linear=True, zero_dy=False):
    q, k, v, w = synth.make(wl, seed)
    dy = torch.randn(q.shape, generator=torch.Generator().manual_seed(seed + 11)).to(torch.bfloat16)
    if zero_dy:
        dy.zero_()
    mask = make_mask(wl, topk, seed)
    say(f"case {wl.name} B{wl.B} H{wl.H} N{wl.N} bq{wl.blk_q} topk{topk} linear{linear} zero_dy{zero_dy}")
    got = sg.backward(q.cuda(), k.cuda(), v.cuda(), w.cuda(), dy.cuda(), torch.from_numpy(mask).cuda(), topk=topk,
                      blk_q=wl.blk_q, blk_k=wl.blk_k, linear=linear)
    torch.cuda.synchronize()
    return (q, k, v, w, dy, mask), got


def test_backward_single_token():
    # one token: its only key gets P = 1, so dS = 0 (dQ = dK = 0 up to the rounding of LSE and D) and dV = dY;
    # every block is selected, so the linear branch and dW_p vanish
    wl = synth.custom(1, 2, 1, blk_q=64, topk_frac=1.0)
    (q, k, v, w, dy, mask), (dq, dk, dv, dw) = run(wl, 1)
    bound = 1e-5 * float(torch.abs(dy.float()).max()) * float(torch.abs(torch.cat([k, v]).float()).max())
    assert float(torch.abs(dq).max()) <= bound and float(torch.abs(dk).max()) <= bound
    np.testing.assert_array_equal(to_np(dv), to_np(dy))
    assert not to_np(dw).any()


@pytest.mark.parametrize("N,bq,topk", [(40, 128, 1), (40, 64, 0), (129, 64, 1), (129, 128, 2)])
def test_backward_tiny_and_one_row_tails(N, bq, topk):
    # fewer tokens than one key block, and tails of a single row in both block kinds
    wl = synth.custom(1, 2, N, blk_q=bq, topk_frac=0.5)
    case(wl, topk, seed=N)


def test_backward_zero_dy_gives_zero_gradients():
    _, (dq, dk, dv, dw) = run(SMALL["ragged128"], 3, zero_dy=True)
    for g in (dq, dk, dv, dw):
        assert not to_np(g).any()


def test_backward_no_branch_gives_zero_gradients():
    # no block selected and no linear branch: the output is identically zero
    _, (dq, dk, dv, dw) = run(SMALL["ragged64"], 0, linear=False)
    for g in (dq, dk, dv):
        assert not to_np(g).any()
    assert dw is None


# ---------------------------------------------------------------------------------------------------------
# the 720P layer at full size, with the forward's own selection: exact dQ rows on sampled query blocks of two
# heads; with the linear branch off, the invariants of softmax attention (sum_j dK_j = 0 because every row of dS
# sums to zero; sum_j dV_j = sum_i dY_i because every row of P sums to one)
# ---------------------------------------------------------------------------------------------------------
def full_720p(linear):
    wl = synth.workload(3)
    q, k, v, w = synth.make(wl, 0, device="cuda")
    say(f"full-size {wl.name}: forward for the selection")
    _, ex = sg.forward(q, k, v, w, topk=wl.topk, export=True)
    mask = ex["block_idx"][..., :wl.topk].contiguous()
    del ex
    dy = torch.randn(q.shape, device="cuda", generator=torch.Generator(device="cuda").manual_seed(1)).to(torch.bfloat16)
    say(f"full-size {wl.name}: backward (linear {linear})")
    grads = sg.backward(q, k, v, w, dy, mask, topk=wl.topk, linear=linear)
    torch.cuda.synchronize()
    return wl, q, k, v, w, dy, mask, grads


def test_backward_full_size_720p_dq_blocks():
    wl, q, k, v, w, dy, mask, (dq, dk, dv, dw) = full_720p(True)
    rng = np.random.default_rng(3)
    for (b, h) in [(0, 0), (1, 39)]:
        blocks = sorted({0, wl.n_qb - 1, *rng.choice(wl.n_qb, 3, replace=False).tolist()})
        ref = ob.dq_blocks(to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h]), to_np(w), mask[b, h].cpu().numpy(),
                           to_np(dy[b, h]), wl.blk_q, wl.blk_k, blocks)
        for I in blocks:
            r0, r1 = I * wl.blk_q, min(wl.N, (I + 1) * wl.blk_q)
            close(f"b{b} h{h} dq block {I}", to_np(dq[b, h, r0:r1]), ref[I])
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all() and torch.isfinite(dw).all()


def test_backward_full_size_720p_softmax_invariants():
    wl, q, k, v, w, dy, mask, (dq, dk, dv, dw) = full_720p(False)
    for (b, h) in [(0, 0), (0, 17), (1, 39)]:
        sk = to_np(dk[b, h]).sum(axis=0)
        scale = np.abs(to_np(dk[b, h])).sum(axis=0).max()
        say(f"  b{b} h{h}: |sum dK| / sum |dK| = {np.abs(sk).max() / scale:.2e}")
        assert np.abs(sk).max() <= 1e-4 * scale
        sv, sy = to_np(dv[b, h]).sum(axis=0), to_np(dy[b, h]).sum(axis=0)
        close(f"b{b} h{h} sum dV vs sum dY", sv, sy)


# ---------------------------------------------------------------------------------------------------------
# with the RMSNorm of Q and K before the path: gradients of the raw inputs and of the norm weights
# ---------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,topk", [("ragged128", 3), ("ragged128", 0), ("ragged64", 2)])
def test_backward_with_qk_norm(name, topk):
    wl = SMALL[name]
    q, k, v, w = synth.make(wl, 8)
    gq, gk = synth.make_norm_weights(wl.H, wl.D, 8)
    dy = torch.randn(q.shape, generator=torch.Generator().manual_seed(19)).to(torch.bfloat16)
    mask = make_mask(wl, topk, 8)
    say(f"case norm {wl.name} B{wl.B} H{wl.H} N{wl.N} topk{topk}")
    dq, dk, dv, dw, dgq, dgk = sg.backward(q.cuda(), k.cuda(), v.cuda(), w.cuda(), dy.cuda(),
                                           torch.from_numpy(mask).cuda(), topk=topk, blk_q=wl.blk_q, blk_k=wl.blk_k,
                                           norm=(gq.cuda(), gk.cuda(), synth.NORM_EPS))
    torch.cuda.synchronize()
    rq, rk, rv, rw, rgq, rgk = ob.backward_with_norm(to_np(q), to_np(k), to_np(v), to_np(w), mask, to_np(dy),
                                                     wl.blk_q, wl.blk_k, to_np(gq), to_np(gk), synth.NORM_EPS)
    for b in range(wl.B):
        for h in range(wl.H):
            close(f"b{b} h{h} dq", to_np(dq[b, h]), rq[b, h])
            close(f"b{b} h{h} dk", to_np(dk[b, h]), rk[b, h])
            close(f"b{b} h{h} dv", to_np(dv[b, h]), rv[b, h])
    close("dW_p", to_np(dw), rw)
    close("d gamma_q", to_np(dgq), rgq)
    close("d gamma_k", to_np(dgk), rgk)


def test_backward_full_size_720p_qk_norm_step():
    # the norm step at full size: the backward without the norm on the forward's own normalized Q, K gives the
    # gradient g at the normalized values; the backward with the norm must equal the norm's backward of that g
    # (closed form in fp64 on sampled tokens over all heads; the weight gradients summed over every token)
    wl = synth.workload(3)
    q, k, v, w = synth.make(wl, 0, device="cuda")
    gq, gk = synth.make_norm_weights(wl.H, wl.D, 0, device="cuda")
    eps = synth.NORM_EPS
    say(f"full-size {wl.name} with the norm: forward")
    _, ex = sg.forward(q, k, v, w, topk=wl.topk, export=True, norm=(gq, gk, eps))
    sel = ex["block_idx"][..., :wl.topk].contiguous()
    qh, kh = ex["q_hat"], ex["k_hat"]
    del ex
    dy = torch.randn(q.shape, device="cuda", generator=torch.Generator(device="cuda").manual_seed(1)).to(torch.bfloat16)
    say("backward with the norm")
    dq, dk, dv, dw, dgq, dgk = sg.backward(q, k, v, w, dy, sel, topk=wl.topk, norm=(gq, gk, eps))
    say("backward at the normalized values")
    gq_, gk_, dv2, dw2, = sg.backward(qh, kh, v, w, dy, sel, topk=wl.topk)
    torch.cuda.synchronize()
    assert torch.equal(dv, dv2) and torch.equal(dw, dw2)
    n = wl.H * wl.D
    rng = np.random.default_rng(2)
    for x, g, wt, dx, dwt, name in ((q, gq_, gq, dq, dgq, "q"), (k, gk_, gk, dk, dgk, "k")):
        X = x.double().permute(0, 2, 1, 3).reshape(wl.B, wl.N, n)      # token-major [B, N, H*D]
        G = g.double().permute(0, 2, 1, 3).reshape(wl.B, wl.N, n)
        W = wt.double().reshape(1, 1, n)
        r = 1.0 / torch.sqrt((X * X).sum(-1, keepdim=True) / n + float(np.float32(eps)))
        want_dw = (X * r * G).sum(dim=(0, 1))
        close(f"d gamma_{name}", to_np(dwt), want_dw.cpu().numpy())
        for _ in range(6):
            b, t = int(rng.integers(wl.B)), int(rng.integers(wl.N))
            xs, gs, rs = X[b, t], G[b, t], r[b, t]
            s = (xs * W[0, 0] * gs).sum()
            want = rs * W[0, 0] * gs - xs * rs ** 3 * s / n
            got = dx[b, :, t, :].double().reshape(n)
            close(f"d{name} token ({b}, {t})", got.cpu().numpy(), want.cpu().numpy())
