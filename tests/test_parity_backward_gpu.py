"""GPU parity of the SLA backward (sagesla_backward) with the fp64 oracle (oracle/sla_backward.py) on seeded
inputs and seeded selections.

Bar, derived from the precision the forward itself runs at. The forward rounds its probabilities P to bf16 before
the PV product; the backward does the same with P (in dV = P^T dY) and with dS = P (dP - D) (in dQ = dS K and
dK = dS^T Q), each rounded once to nearest (relative error <= 2^-9), every other operand being an exact bf16
input, and accumulates in fp32. An element of such a product sum_k a_k b_k is then off by at most
2^-9 sum_k |a_k| |b_k| from rounding plus the fp32 accumulation of at most ~10^4 terms (gamma_n < 2^-11). So each
element of dQ, dK and dV must satisfy
    |got - exact| <= 2^-8 * T + FLOOR * max|exact|,
with T the fp64 magnitude term of its product (sm |dS| |K|, sm |dS|^T |Q| or P^T |dY|, computed here from the
exact P and dS of the selection) and FLOOR = 1e-4 for the fp32 steps before the rounding (scores, exp2, D) and
for the linear branch, which keeps bf16 hi + lo operands (~2^-16 per product) but divides by den and cancels in
G + dden Z_m: it reaches 2.6e-5 of the largest magnitude on its own (the linear-only case).
dW_p comes from the linear branch alone: relative L2 error <= 1e-4, max-abs <= 1e-3 of its largest magnitude.
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
U = 2.0 ** -8   # bf16 rounding of P and dS (2^-9) plus fp32 accumulation, with margin
FLOOR = 1e-4


def say(*a):
    print(*a, flush=True)


def close(name, got, want):
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    mx = np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-300)
    say(f"    {name}: rel-L2 {rel:.2e}, max-abs/max {mx:.2e}")
    assert rel <= REL_L2 and mx <= MAX_REL, f"{name}: rel-L2 {rel:.3e} max {mx:.3e}"


def sparse_terms(Q, K, V, dY, idx, blk_q, blk_k, sm_scale=None, blocks=None):
    """fp64 magnitude terms of one head's sparse-branch products: TdQ = sm |dS| |K|, TdK = sm |dS|^T |Q|,
    TdV = P^T |dY| ([N, D] each) and R[i] = sum_j |dS_ij|, from the exact P = softmax(q . k sm) over the selected
    keys of each row and dS = P (dP - D), dP = dY V^T, D = sum_j P dP. `blocks` limits the work to those query
    blocks (their TdQ rows and R; TdK, TdV then hold only their contributions)."""
    Q, K, V, dY = (np.asarray(a, np.float64) for a in (Q, K, V, dY))
    N, D = Q.shape
    sm = 1.0 / np.sqrt(D) if sm_scale is None else sm_scale
    n_qb, n_kb = (N + blk_q - 1) // blk_q, (N + blk_k - 1) // blk_k
    TdQ, TdK, TdV, R = np.zeros((N, D)), np.zeros((N, D)), np.zeros((N, D)), np.zeros(N)
    for I in (range(n_qb) if blocks is None else blocks):
        sel = sorted(set(int(J) for J in idx[I]))
        if not sel:
            continue
        r0, r1 = I * blk_q, min(N, (I + 1) * blk_q)
        keys = np.concatenate([np.arange(J * blk_k, min(N, (J + 1) * blk_k)) for J in sel])
        S = Q[r0:r1] @ K[keys].T * sm
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dP = dY[r0:r1] @ V[keys].T
        dS = np.abs(P * (dP - (P * dP).sum(axis=1, keepdims=True)))
        TdQ[r0:r1] = sm * dS @ np.abs(K[keys])
        TdK[keys] += sm * dS.T @ np.abs(Q[r0:r1])
        TdV[keys] += P.T @ np.abs(dY[r0:r1])
        R[r0:r1] = dS.sum(axis=1)
    return TdQ, TdK, TdV, R


def within(name, got, want, T):
    """every element within 2^-8 T + FLOOR max|want| of the exact value (T: the product's magnitude term)"""
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    err = np.abs(got - want)
    lim = U * np.asarray(T, np.float64) + FLOOR * max(np.abs(want).max(), 1e-300)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    worst = float((err / lim).max())
    say(f"    {name}: rel-L2 {rel:.2e}, max err/bound {worst:.3f}")
    assert worst <= 1.0, f"{name}: error reaches {worst:.3f} of the bound"


def make_mask(wl, topk, seed):
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(wl.B * wl.H * wl.n_qb):
        r = np.sort(rng.choice(wl.n_kb, topk, replace=False)) if topk else np.zeros(0, np.int64)
        rows.append(r)
    return np.stack(rows).reshape(wl.B, wl.H, wl.n_qb, topk).astype(np.int32)


def case(wl, topk, linear=True, seed=0, sm_scale=0.0, qk_mul=1.0):
    q, k, v, w = synth.make(wl, seed)
    if qk_mul != 1.0:
        q, k = ((t.float() * qk_mul).to(torch.bfloat16) for t in (q, k))
    dy = (torch.randn(q.shape, generator=torch.Generator().manual_seed(seed + 11))).to(torch.bfloat16)
    mask = make_mask(wl, topk, seed)
    say(f"case {wl.name} B{wl.B} H{wl.H} N{wl.N} bq{wl.blk_q} topk{topk} linear{linear} sm_scale{sm_scale}")
    dq, dk, dv, dw = sg.backward(q.cuda(), k.cuda(), v.cuda(), w.cuda(), dy.cuda(), torch.from_numpy(mask).cuda(),
                                 topk=topk, blk_q=wl.blk_q, blk_k=wl.blk_k, linear=linear, sm_scale=sm_scale)
    torch.cuda.synchronize()
    sm = sm_scale if sm_scale > 0 else None
    rq, rk, rv, rw = ob.backward(to_np(q), to_np(k), to_np(v), to_np(w), mask, to_np(dy), wl.blk_q, wl.blk_k,
                                 linear=linear, sm_scale=sm)
    for b in range(wl.B):
        for h in range(wl.H):
            say(f"  b{b} h{h}")
            tq, tk, tv, _ = sparse_terms(to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h]), to_np(dy[b, h]), mask[b, h],
                                         wl.blk_q, wl.blk_k, sm_scale=sm)
            within("dq", to_np(dq[b, h]), rq[b, h], tq)
            within("dk", to_np(dk[b, h]), rk[b, h], tk)
            within("dv", to_np(dv[b, h]), rv[b, h], tv)
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


@pytest.mark.parametrize("name", list(SMALL))
def test_backward_power_of_two_scaling(name):
    # exact for the arithmetic of the backward: dY times 4 scales dP, D, dS, their bf16 roundings, every product and
    # sum by a power of two, so dQ, dK, dV and dW_p must be 4 times the unscaled ones bit for bit
    wl = SMALL[name]
    q, k, v, w = (t.cuda() for t in synth.make(wl, 12))
    dy = torch.randn(q.shape, generator=torch.Generator().manual_seed(13)).to(torch.bfloat16).cuda()
    mask = torch.from_numpy(make_mask(wl, 2, 12)).cuda()
    g1 = sg.backward(q, k, v, w, dy, mask, topk=2, blk_q=wl.blk_q, blk_k=wl.blk_k)
    g2 = sg.backward(q, k, v, w, (dy.float() * 4).to(torch.bfloat16), mask, topk=2, blk_q=wl.blk_q, blk_k=wl.blk_k)
    torch.cuda.synchronize()
    for name_, a, b in zip(("dq", "dk", "dv", "dw"), g1, g2):
        assert torch.equal(b, a * 4), name_


def test_backward_heads_are_independent():
    # exact: dQ, dK, dV of a (b, h) slice depend on that slice alone, so permuting the heads permutes them bit for bit
    # (dW_p is a sum over heads in a fixed order, so only its value is checked)
    wl = synth.custom(1, 3, 700, blk_q=128, topk_frac=0.3)
    q, k, v, w = (t.cuda() for t in synth.make(wl, 15))
    dy = torch.randn(q.shape, generator=torch.Generator().manual_seed(16)).to(torch.bfloat16).cuda()
    mask = torch.from_numpy(make_mask(wl, 3, 15)).cuda()
    g = sg.backward(q, k, v, w, dy, mask, topk=3, blk_q=wl.blk_q, blk_k=wl.blk_k)
    perm = torch.tensor([1, 2, 0], device="cuda")
    pc = lambda t: t[:, perm].contiguous()
    gp = sg.backward(pc(q), pc(k), pc(v), w, pc(dy), pc(mask), topk=3, blk_q=wl.blk_q, blk_k=wl.blk_k)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g[:3], gp[:3]):
        assert torch.equal(b, a[:, perm]), name
    assert torch.allclose(gp[3], g[3], rtol=1e-5, atol=1e-6 * float(g[3].abs().max()))


@pytest.mark.parametrize("qk_mul", [8.0, 1.0 / 16])
def test_backward_large_and_small_qk(qk_mul):
    # Q and K scaled by 8 (sharp rows, phi(K) large in the linear branch) and by 1/16 (flat rows)
    case(SMALL["ragged128"], 3, qk_mul=qk_mul)


@pytest.mark.parametrize("sm_scale", [0.02, 0.5])
def test_backward_softmax_scales(sm_scale):
    # softmax scales other than 1/sqrt(D): a flatter and a sharper P
    case(SMALL["ragged128"], 3, sm_scale=sm_scale)


def test_backward_sparse_only():
    case(SMALL["ragged128"], 3, linear=False)


def test_backward_linear_only():
    case(SMALL["ragged128"], 0)


def test_backward_all_selected():
    wl = SMALL["ragged64"]
    case(wl, wl.n_kb)


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
def full_720p(linear, wl=None):
    wl = synth.workload(3) if wl is None else wl
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


def test_backward_full_size_720p_dq_blocks(wl=None, heads=((0, 0), (1, 39))):
    wl, q, k, v, w, dy, mask, (dq, dk, dv, dw) = full_720p(True, wl)
    rng = np.random.default_rng(3)
    for (b, h) in heads:
        blocks = sorted({0, wl.n_qb - 1, *rng.choice(wl.n_qb, 3, replace=False).tolist()})
        sel = mask[b, h].cpu().numpy()
        ref = ob.dq_blocks(to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h]), to_np(w), sel, to_np(dy[b, h]), wl.blk_q,
                           wl.blk_k, blocks)
        tq = sparse_terms(to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h]), to_np(dy[b, h]), sel, wl.blk_q, wl.blk_k,
                          blocks=blocks)[0]
        for I in blocks:
            r0, r1 = I * wl.blk_q, min(wl.N, (I + 1) * wl.blk_q)
            within(f"b{b} h{h} dq block {I}", to_np(dq[b, h, r0:r1]), ref[I], tq[r0:r1])
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all() and torch.isfinite(dw).all()


def test_backward_full_size_720p_softmax_invariants(wl=None, heads=((0, 0), (0, 17), (1, 39))):
    # exact: sum_j dK_j = sm sum_i q_i sum_j dS_ij = 0 and sum_j dV_j = sum_i dY_i sum_j P_ij = sum_i dY_i. With dS and
    # P rounded to bf16 (<= 2^-9 each) the sums are off by at most 2^-9 sm sum_i |q_i| R_i (R_i = sum_j |dS_ij|) and
    # 2^-9 sum_i |dY_i| (the rows of P sum to one), checked at 2^-8 plus the fp32 floor
    wl, q, k, v, w, dy, mask, (dq, dk, dv, dw) = full_720p(False, wl)
    sm = 1.0 / np.sqrt(wl.D)
    for (b, h) in heads:
        Q, Y = to_np(q[b, h]).astype(np.float64), to_np(dy[b, h]).astype(np.float64)
        R = sparse_terms(Q, to_np(k[b, h]), to_np(v[b, h]), Y, mask[b, h].cpu().numpy(), wl.blk_q, wl.blk_k)[3]
        sk = to_np(dk[b, h]).astype(np.float64).sum(axis=0)
        lim_k = U * sm * (np.abs(Q) * R[:, None]).sum(axis=0) + FLOOR * np.abs(to_np(dk[b, h])).max()
        say(f"  b{b} h{h}: |sum dK| / bound = {np.max(np.abs(sk) / lim_k):.3f}")
        assert np.all(np.abs(sk) <= lim_k)
        sv, sy = to_np(dv[b, h]).astype(np.float64).sum(axis=0), Y.sum(axis=0)
        lim_v = U * np.abs(Y).sum(axis=0) + FLOOR * np.abs(sy).max()
        say(f"  b{b} h{h}: |sum dV - sum dY| / bound = {np.max(np.abs(sv - sy) / lim_v):.3f}")
        assert np.all(np.abs(sv - sy) <= lim_v)


WL_720P_B8 = synth.custom(8, 40, 75600, grid=(21, 45, 80), structured=True, blk_q=128, topk_frac=0.1, name="720p-b8")


@pytest.mark.timeout(600)
def test_backward_large_batch():
    # the 720P layer at batch 8, 3.1e9 elements per tensor (past 32-bit offsets): the exact dQ rows of sampled query
    # blocks with the linear branch on, then the softmax identities of dK and dV with it off, on the first and the
    # last head
    assert WL_720P_B8.B * WL_720P_B8.H * WL_720P_B8.N * WL_720P_B8.D > 2 ** 31
    test_backward_full_size_720p_dq_blocks(WL_720P_B8, ((0, 0), (7, 39)))
    torch.cuda.empty_cache()
    test_backward_full_size_720p_softmax_invariants(WL_720P_B8, ((0, 0), (7, 39)))


@pytest.mark.timeout(600)
def test_backward_max_key_blocks():
    # the largest key-block count (20480 blocks, N = 1310697, 2048-entry selections, bitmaps of 320 and 640 words):
    # the exact dQ rows of sampled query blocks with the linear branch on
    wl = synth.custom(1, 1, 20480 * 64 - 23, blk_q=128, topk_frac=0.1, name="max-key-blocks")
    assert wl.n_kb == 20480 and wl.topk == 2048
    test_backward_full_size_720p_dq_blocks(wl, ((0, 0),))


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
    # the attention's error bound at the normalized values (E = 2^-8 T + FLOOR max|g| for g = dQ-hat, dK-hat), carried
    # through the norm's Jacobian in absolute values: per token, with r and the weights w over its H*D channels,
    #   |d dx_c| <= r |w_c| E_c + |x_c| r^3 / n sum_c' |x_c'| |w_c'| E_c',   |d dgamma_c| <= sum_tokens |x_c| r E_c
    from oracle.sagesla import qk_rmsnorm
    X = {"q": to_np(q).astype(np.float64), "k": to_np(k).astype(np.float64)}
    Xh = {n: np.stack([qk_rmsnorm(X[n][b], to_np(gm), synth.NORM_EPS)[0] for b in range(wl.B)])
          for n, gm in (("q", gq), ("k", gk))}
    gh_q, gh_k = ob.backward(Xh["q"], Xh["k"], to_np(v), to_np(w), mask, to_np(dy), wl.blk_q, wl.blk_k)[:2]
    E = {"q": np.zeros_like(X["q"]), "k": np.zeros_like(X["k"])}
    for b in range(wl.B):
        for h in range(wl.H):
            tq, tk, _, _ = sparse_terms(Xh["q"][b, h], Xh["k"][b, h], to_np(v[b, h]), to_np(dy[b, h]), mask[b, h],
                                        wl.blk_q, wl.blk_k)
            E["q"][b, h] = U * tq + FLOOR * np.abs(gh_q[b, h]).max()
            E["k"][b, h] = U * tk + FLOOR * np.abs(gh_k[b, h]).max()
    n = wl.H * wl.D
    lim, limw = {}, {}
    for name, gm in (("q", gq), ("k", gk)):
        x = X[name].transpose(0, 2, 1, 3).reshape(wl.B, wl.N, n)
        e = E[name].transpose(0, 2, 1, 3).reshape(wl.B, wl.N, n)
        wv = np.abs(to_np(gm).astype(np.float64)).reshape(1, 1, n)
        r = 1.0 / np.sqrt((x * x).sum(-1, keepdims=True) / n + float(np.float32(synth.NORM_EPS)))
        bd = r * wv * e + np.abs(x) * r ** 3 / n * (np.abs(x) * wv * e).sum(-1, keepdims=True)
        lim[name] = bd.reshape(wl.B, wl.N, wl.H, wl.D).transpose(0, 2, 1, 3)
        limw[name] = (np.abs(x) * r * e).sum(axis=(0, 1))
    for b in range(wl.B):
        for h in range(wl.H):
            within(f"b{b} h{h} dq", to_np(dq[b, h]), rq[b, h], lim["q"][b, h] / U)
            within(f"b{b} h{h} dk", to_np(dk[b, h]), rk[b, h], lim["k"][b, h] / U)
            tv = sparse_terms(Xh["q"][b, h], Xh["k"][b, h], to_np(v[b, h]), to_np(dy[b, h]), mask[b, h], wl.blk_q,
                              wl.blk_k)[2]
            within(f"b{b} h{h} dv", to_np(dv[b, h]), rv[b, h], tv)
    close("dW_p", to_np(dw), rw)
    within("d gamma_q", to_np(dgq), rgq, limw["q"] / U)
    within("d gamma_k", to_np(dgk), rgk, limw["k"] / U)


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


@pytest.mark.parametrize("bq,N", [(128, 9000), (64, 5000)], ids=["bq128-N9000", "bq64-N5000"])
def test_backward_many_blocks(bq, N):
    # more than 64 query and key blocks: the selection bitmaps and the transposed keep mask span several 32-bit
    # words on both axes (71 x 141 and 79 x 79 blocks), 10% of the key blocks selected, linear branch on
    wl = synth.custom(1, 1, N, blk_q=bq, topk_frac=0.1)
    assert wl.n_qb > 64 and wl.n_kb > 64
    case(wl, wl.topk, seed=3)


def test_backward_many_blocks_linear_only():
    wl = synth.custom(1, 1, 9000, blk_q=128)
    case(wl, 0, seed=4)
