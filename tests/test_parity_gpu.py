"""Parity of the HIP path (through the C ABI) with the fp64 oracle, element by element, on seeded inputs.

Bars: INT8 codes, scales and the K mean bit-exact; the block mask bit-exact except in near-tie rows (oracle
gap between the k-th and (k+1)-th score below 1e-6, flagged not failed); outputs, computed by the oracle
with the GPU's own mask, within max-abs 2e-2 and cosine >= 0.999; the linear branch gated separately
(cosine >= 0.999, relative L2 <= 1e-3) because its contribution is small next to the output tolerance.
"""
import math
import sys

import numpy as np
import pytest
import torch

import int8_block_sparse_amd as sg
import synth
from oracle import sagesla as orc
from conftest import to_np

pytestmark = pytest.mark.gpu

OUT_ATOL = 2e-2
OUT_COS = 0.999
LIN_COS = 0.999
LIN_REL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    sg.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cos(a, b):
    a, b = a.ravel(), b.ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def run_gpu(q, k, v, w, wl, topk, **kw):
    torch.cuda.synchronize()
    out, ex = sg.forward(q, k, v, w, topk=topk, blk_q=wl.blk_q, blk_k=wl.blk_k, export=True, **kw)
    torch.cuda.synchronize()
    return out, ex


def check_quant(ex, r, b, h):
    assert np.array_equal(ex["q_i8"][b, h].cpu().numpy(), r["q_codes"]), "Q codes differ"
    assert np.array_equal(ex["k_i8"][b, h].cpu().numpy(), r["k_codes"]), "K codes differ"
    assert np.array_equal(ex["q_scale"][b, h].cpu().numpy(), r["q_scales"].astype(np.float32)), "Q scales differ"
    assert np.array_equal(ex["k_scale"][b, h].cpu().numpy(), r["k_scales"].astype(np.float32)), "K scales differ"
    assert np.array_equal(ex["k_mean"][b, h].cpu().numpy(), r["mu"].astype(np.float32)), "K mean differs"
    np.testing.assert_allclose(ex["q_pool"][b, h].cpu().numpy(), r["q_pool"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ex["k_pool"][b, h].cpu().numpy(), r["k_pool"], rtol=1e-10, atol=1e-13)


def check_mask(gidx, r, topk):
    """Bit-exact mask except near-tie rows; returns the number of flagged rows."""
    want = r["idx"]
    got = gidx[:, :topk] if topk else np.zeros((want.shape[0], 0), np.int32)
    flagged = 0
    for I in range(want.shape[0]):
        if np.array_equal(got[I], want[I]):
            continue
        assert r["gap"][I] < orc.NEAR_TIE, f"mask row {I} differs with gap {r['gap'][I]:.3e}"
        flagged += 1
        assert np.all(np.diff(got[I]) > 0), "GPU row not ascending/unique"
    return flagged


def check_scores(ex, r, b, h):
    """The exported fp64 block scores against the oracle's, within the rounding bound of the two fp64 sums
    (2^-44 |q_pool| . |k_pool|; the kernel's sums skip the oracle's 1/sqrt(D)). Returns the largest difference
    as a fraction of that bound (0 when the selection did not run)."""
    if "scores" not in ex:
        return 0.0
    D = r["q_pool"].shape[1]
    got = ex["scores"][b, h].cpu().numpy() / math.sqrt(D)
    bound = 2.0 ** -44 * (np.abs(r["q_pool"]) @ np.abs(r["k_pool"]).T) / math.sqrt(D) + 1e-300
    ratio = float((np.abs(got - r["scores"]) / bound).max())
    assert ratio <= 1.0, f"block scores off by {ratio:.2f} of their rounding bound"
    return ratio


def bf16_half_ulp(x):
    """Half the bf16 spacing at |x| (8 significant bits)."""
    e = np.frexp(np.maximum(np.abs(x), 2.0 ** -126))[1]
    return np.ldexp(1.0, e - 9)


def check_out(out, r, rows=None, lin=None, bf16_bound=False):
    """max-abs <= 2e-2 and cosine >= 0.999; with bf16_bound the allowance grows by the bf16 half-ulp of the
    expected value (outputs beyond |8| cannot be stored in bf16 closer than 2e-2)."""
    o = out if rows is None else out[rows]
    want = r["out"] if rows is None else r["out"][rows]
    excess = np.abs(o - want) - (bf16_half_ulp(want) if bf16_bound else 0.0)
    err = excess.max()
    c = cos(o, want)
    if not (err <= OUT_ATOL and c >= OUT_COS):
        if lin is not None:
            lg = lin if rows is None else lin[rows]
            lw = r["o_lin"] if rows is None else r["o_lin"][rows]
            ws = r["o_s"] if rows is None else r["o_s"][rows]
            say(f"    diag: sparse part max-abs {np.abs(o - lg - ws).max():.3e} cos {cos(o - lg, ws):.6f}; "
                f"linear part max-abs {np.abs(lg - lw).max():.3e} cos {cos(lg, lw):.6f}")
        bad = np.argwhere(np.abs(o - want) > OUT_ATOL)
        say(f"    diag: {len(bad)} elements over tolerance, first rows {np.unique(bad[:, 0])[:16]}")
    assert err <= OUT_ATOL and c >= OUT_COS, f"out max-abs {err:.3e} cos {c:.6f}"
    if lin is not None:
        lw = r["o_lin"] if rows is None else r["o_lin"][rows]
        lg = lin if rows is None else lin[rows]
        if np.abs(lw).max() == 0:
            assert np.abs(lg).max() == 0
        else:
            rel = np.linalg.norm(lg - lw) / np.linalg.norm(lw)
            assert cos(lg, lw) >= LIN_COS and rel <= LIN_REL, f"o_lin cos {cos(lg, lw):.6f} rel {rel:.3e}"
    return err, c


def oracle_norm(x, b, gamma, chunk=4096):
    """The oracle's RMSNorm of batch entry b of x ([B, H, N, D], any device), token chunk by token chunk (each
    token's scale depends on all its heads only). Returns (normalized [H, N, D] fp64, True when no token's scale
    rounding is ambiguous: the seeded inputs are checked to have none)."""
    H, N, D = x.shape[1:]
    y = np.empty((H, N, D))
    clear = True
    for n0 in range(0, N, chunk):
        yc, _, amb = orc.qk_rmsnorm(to_np(x[b, :, n0:n0 + chunk]), to_np(gamma), synth.NORM_EPS)
        y[:, n0:n0 + chunk] = yc
        clear &= not amb.any()
    return y, clear


def check_hat(ex, b, h, want, name):
    got = to_np(ex[name][b, h])
    assert np.array_equal(got, want), f"{name}: {np.sum(got != want)} normalized values differ"


def full_case(wl, seed=0, topk=None, linear=None, smooth_k=True, w_mul=1.0, prep=None, group32=False, norm=False,
              sm_scale=0.0):
    topk = wl.topk if topk is None else topk
    linear = wl.linear if linear is None else linear
    q, k, v, w = synth.make(wl, seed)
    if prep is not None:
        q, k, v = prep(q, k, v)
    w = (w.float() * w_mul).to(torch.bfloat16)
    dq, dk, dv, dw = (t.cuda() for t in (q, k, v, w))
    say(f"case {wl.name} B{wl.B} H{wl.H} N{wl.N} bq{wl.blk_q} topk{topk} linear{linear} smooth{smooth_k}"
        f" group32{group32} norm{norm} sm_scale{sm_scale}")
    nw = synth.make_norm_weights(wl.H, wl.D, seed) if norm else None
    out, ex = run_gpu(dq, dk, dv, dw, wl, topk, linear=linear, smooth_k=smooth_k, group32=group32,
                      norm=(nw[0].cuda(), nw[1].cuda(), synth.NORM_EPS) if norm else None, sm_scale=sm_scale)
    sm = sm_scale if sm_scale > 0 else None
    qg = 32 if group32 else None
    outn = to_np(out)
    W = to_np(w)
    flagged = 0
    for b in range(wl.B):
        if norm:
            qh, eq = oracle_norm(q, b, nw[0])
            kh, ek = oracle_norm(k, b, nw[1])
            assert eq and ek
        for h in range(wl.H):
            Q, K, V = to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h])
            if norm:
                Q, K = qh[h], kh[h]
                check_hat(ex, b, h, Q, "q_hat")
                check_hat(ex, b, h, K, "k_hat")
            gidx = ex["block_idx"][b, h].cpu().numpy()
            r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, topk, linear=linear, smooth_k=smooth_k,
                                 quant_group=qg, sm_scale=sm)
            assert r["exact_sum_ok"]
            check_quant(ex, r, b, h)
            check_scores(ex, r, b, h)
            flagged += check_mask(gidx, r, topk)
            rg = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, topk, linear=linear, smooth_k=smooth_k,
                                  mask=gidx[:, :topk] if topk else np.zeros((wl.n_qb, 0), np.int32),
                                  quant_group=qg, sm_scale=sm)
            lin = to_np(ex["o_lin"][b, h]) if linear else None
            err, c = check_out(outn[b, h], rg, lin=lin, bf16_bound=w_mul != 1.0)
            say(f"  b{b} h{h}: out max-abs {err:.2e} cos {c:.6f}")
    return flagged


SMALL = {
    "tiny": synth.workload(0),
    "ragged128": synth.custom(1, 2, 1000, blk_q=128, topk_frac=0.2),
    "ragged64": synth.custom(2, 1, 330, blk_q=64, topk_frac=0.34),
    "grid": synth.custom(1, 1, 6 * 20 * 24, grid=(6, 20, 24), structured=True, blk_q=128, topk_frac=0.1),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    assert full_case(SMALL[name]) == 0


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small_group32(name):
    # one INT8 scale per 32 tokens of Q and of K (thread-level granularity)
    assert full_case(SMALL[name], group32=True) == 0


@pytest.mark.parametrize("name", ["tiny", "ragged128", "ragged64"])
def test_forward_small_qk_norm(name):
    # Q and K first normalized by RMSNorm over all heads of each token
    assert full_case(SMALL[name], norm=True) == 0


@pytest.mark.parametrize("N,bq,topk", [(1, 64, 1), (1, 128, 0), (40, 128, 1), (64, 64, 0), (65, 64, 1),
                                        (65, 128, 2), (129, 64, 2), (129, 128, 1)])
@pytest.mark.parametrize("group32", [False, True], ids=["block", "group32"])
def test_forward_tiny_and_one_row_tails(N, bq, topk, group32):
    # a single token, fewer tokens than one key block, exactly one block, and tails of a single row in both block
    # kinds; the list from empty (linear branch only) to every block (no linear branch)
    wl = synth.custom(1, 2, N, blk_q=bq, topk_frac=0.5)
    assert topk <= wl.n_kb
    assert full_case(wl, topk=topk, group32=group32) == 0


@pytest.mark.parametrize("sm_scale", [0.02, 0.5, 2.0])
@pytest.mark.parametrize("group32", [False, True], ids=["block", "group32"])
def test_softmax_scales(sm_scale, group32):
    # softmax scales other than 1/sqrt(D) (0.088): flatter and far sharper rows, which move waves between the
    # bounded shift and the running maximum and blocks between the two exponent forms
    assert full_case(SMALL["ragged128"], sm_scale=sm_scale, group32=group32) == 0


def test_topk_zero_linear_only():
    full_case(SMALL["ragged128"], topk=0)


def test_topk_all_with_linear_is_dense():
    wl = SMALL["ragged128"]
    full_case(wl, topk=wl.n_kb, linear=True)


def test_dense_no_linear():
    wl = synth.custom(1, 2, 777, blk_q=128, topk_frac=1.0, linear=False)
    full_case(wl)


@pytest.mark.parametrize("name,linear", [("ragged128", True), ("ragged64", True), ("ragged64", False)])
def test_options_together(name, linear):
    # every option of the forward at once: the RMSNorm of Q and K, 32-token scales and a softmax scale of 0.5
    assert full_case(SMALL[name], norm=True, group32=True, linear=linear, sm_scale=0.5) == 0


@pytest.mark.parametrize("name", ["ragged128", "ragged64"])
@pytest.mark.parametrize("group32", [False, True], ids=["block", "group32"])
def test_sparse_no_linear(name, group32):
    # the selection without the linear branch: the unselected blocks simply drop out of the output
    assert full_case(SMALL[name], linear=False, group32=group32) == 0


def test_no_smoothing():
    full_case(SMALL["ragged64"], smooth_k=False)


def test_linear_projection_x100():
    # makes the linear branch dominate the output; outputs reach |8|+, so the bf16 storage bound applies
    full_case(SMALL["ragged128"], w_mul=100.0)


def test_zero_and_constant_blocks():
    def prep(q, k, v):
        q = q.clone()
        k = k.clone()
        q[:, :, 128:256] = 0  # an all-zero query block: scale 0, codes 0
        k[:, :, 64:128] = k[:, :, 64:65]  # a key block of identical rows
        k[:, :, :, 5] = 0.75  # a constant channel: smoothed to exactly 0
        return q, k, v
    full_case(SMALL["ragged128"], prep=prep)


@pytest.mark.parametrize("mul", [32.0, 1.0 / 64])
@pytest.mark.parametrize("group32", [False, True], ids=["block", "group32"])
def test_large_and_small_qk(mul, group32):
    # Q and K scaled by 32 (scores 1024 times larger: near one-hot rows, the running maximum and the two-instruction
    # exponent form everywhere, phi(K) up to ~130 in the state table) and by 1/64 (almost flat rows)
    def prep(q, k, v):
        return (q.float() * mul).to(torch.bfloat16), (k.float() * mul).to(torch.bfloat16), v
    # (scaled by 1/64 the pooled scores come within 1e-6 of each other: mask rows may differ there, flagged)
    full_case(SMALL["ragged128"], prep=prep, group32=group32)


@pytest.mark.parametrize("name", ["ragged128", "ragged64"])
@pytest.mark.parametrize("group32", [False, True], ids=["block", "group32"])
def test_v_power_of_two_scaling(name, group32):
    # exact for any arithmetic of the path: V times 2^2 leaves the codes, scales, selection and probabilities as
    # they are, and every later product, sum, per-block exponent and rounding scales by exactly 2^2, so the outputs
    # (and the linear branch's) must be 4 times the unscaled ones bit for bit
    wl = SMALL[name]
    q, k, v, w = (t.cuda() for t in synth.make(wl, 6))
    o1, e1 = run_gpu(q, k, v, w, wl, wl.topk, group32=group32)
    o2, e2 = run_gpu(q, k, (v.float() * 4).to(torch.bfloat16), w, wl, wl.topk, group32=group32)
    assert torch.equal(o2.float(), o1.float() * 4)
    assert torch.equal(e2["o_lin"], e1["o_lin"] * 4)
    assert torch.equal(e2["block_idx"], e1["block_idx"])


def test_heads_and_batch_entries_are_independent():
    # exact: every (b, h) slice is computed on its own (W_p is shared, nothing else), so permuting the heads or
    # running one batch entry alone must reproduce the corresponding slices bit for bit
    wl = synth.custom(2, 3, 700, blk_q=128, topk_frac=0.3)
    q, k, v, w = (t.cuda() for t in synth.make(wl, 14))
    o, e = run_gpu(q, k, v, w, wl, wl.topk)
    perm = torch.tensor([2, 0, 1], device="cuda")
    op, ep = run_gpu(q[:, perm].contiguous(), k[:, perm].contiguous(), v[:, perm].contiguous(), w, wl, wl.topk)
    assert torch.equal(op, o[:, perm]) and torch.equal(ep["block_idx"], e["block_idx"][:, perm])
    wl1 = synth.custom(1, 3, 700, blk_q=128, topk_frac=0.3)
    o1, e1 = run_gpu(q[1:].contiguous(), k[1:].contiguous(), v[1:].contiguous(), w, wl1, wl.topk)
    assert torch.equal(o1, o[1:]) and torch.equal(e1["o_lin"], e["o_lin"][1:])


def test_given_mask_matches_oracle_with_same_mask():
    wl = SMALL["ragged128"]
    q, k, v, w = synth.make(wl, 3)
    rng = np.random.default_rng(5)
    topk = 4
    mask = np.stack([np.sort(rng.choice(wl.n_kb, topk, replace=False)) for _ in range(wl.B * wl.H * wl.n_qb)])
    mask = mask.reshape(wl.B, wl.H, wl.n_qb, topk).astype(np.int32)
    dmask = torch.from_numpy(mask).cuda()
    out, ex = run_gpu(q.cuda(), k.cuda(), v.cuda(), w.cuda(), wl, topk, mask=dmask)
    for h in range(wl.H):
        r = orc.forward_head(to_np(q[0, h]), to_np(k[0, h]), to_np(v[0, h]), to_np(w), wl.blk_q, wl.blk_k, topk,
                             mask=mask[0, h])
        check_out(to_np(out[0, h]), r, lin=to_np(ex["o_lin"][0, h]))


@pytest.mark.parametrize("group32", [False, True], ids=["block", "group32"])
def test_given_mask_ragged_block_first(group32):
    # caller-given lists in descending order that hold the ragged last key block first: the attention kernel's
    # generic loop (the ring assumes the ragged block can only come last)
    wl = SMALL["ragged128"]
    q, k, v, w = synth.make(wl, 4)
    rng = np.random.default_rng(6)
    topk = 5
    rows = []
    for _ in range(wl.B * wl.H * wl.n_qb):
        others = rng.choice(wl.n_kb - 1, topk - 1, replace=False)
        rows.append(np.sort(np.append(others, wl.n_kb - 1))[::-1])
    mask = np.stack(rows).reshape(wl.B, wl.H, wl.n_qb, topk).astype(np.int32)
    out, ex = run_gpu(q.cuda(), k.cuda(), v.cuda(), w.cuda(), wl, topk, mask=torch.from_numpy(mask).cuda(),
                      group32=group32)
    for h in range(wl.H):
        r = orc.forward_head(to_np(q[0, h]), to_np(k[0, h]), to_np(v[0, h]), to_np(w), wl.blk_q, wl.blk_k, topk,
                             mask=mask[0, h], quant_group=32 if group32 else None)
        check_out(to_np(out[0, h]), r, lin=to_np(ex["o_lin"][0, h]))


@pytest.mark.parametrize("group32", [False, True], ids=["block", "group32"])
def test_bounded_shift_and_running_max_paths(group32):
    # The attention kernel subtracts a per-row bound of the scores (Cauchy-Schwarz over the codes) instead of a
    # running max when that bound lies within kBoundGap of a known score of the row; query block 1, scaled by 64,
    # has its scores and their bound scaled alike, so its gap is far beyond and its waves keep the lazy running
    # max, while the other blocks take the bounded shift. Lists of one block keep the running max too.
    wl = SMALL["ragged128"]
    q, k, v, w = synth.make(wl, 7)
    q = q.clone()
    q[:, :, 128:256] = (q[:, :, 128:256].float() * 64).to(torch.bfloat16)
    c0 = math.log2(math.e) / math.sqrt(wl.D)
    for topk in (wl.topk, 1):
        out, ex = run_gpu(q.cuda(), k.cuda(), v.cuda(), w.cuda(), wl, topk, group32=group32)
        for h in range(wl.H):
            gidx = ex["block_idx"][0, h].cpu().numpy()[:, :topk]
            if topk > 1:  # the gaps that decide each wave's path, from the exported codes and scales
                qc = ex["q_i8"][0, h].cpu().numpy().astype(np.int64)
                kc = ex["k_i8"][0, h].cpu().numpy().astype(np.int64)
                qsc = ex["q_scale"][0, h].cpu().numpy().astype(np.float64)
                ksc = ex["k_scale"][0, h].cpu().numpy().astype(np.float64)
                per = 32 if group32 else wl.blk_k
                kn = np.sqrt((kc ** 2).sum(1))
                for I in range(wl.n_qb):
                    rows = np.arange(I * wl.blk_q, min((I + 1) * wl.blk_q, wl.N))
                    cq = (qsc[rows // 32] if group32 else qsc[I]) * c0
                    keys = np.concatenate([np.arange(J * wl.blk_k, min((J + 1) * wl.blk_k, wl.N)) for J in gidx[I]])
                    bound = np.sqrt((qc[rows] ** 2).sum(1)) * cq * (ksc[keys // per] * kn[keys]).max()
                    j0 = gidx[I][0] * wl.blk_k
                    gap = bound - (qc[rows] @ kc[j0]) * cq * ksc[j0 // per]
                    if I == 1:
                        assert gap.max() > 2 * 160, f"block 1 gap {gap.max():.1f}: its waves must keep the running max"
                    else:
                        assert gap.max() < 0.9 * 160, f"block {I} gap {gap.max():.1f}: expected the bounded shift"
            r = orc.forward_head(to_np(q[0, h]), to_np(k[0, h]), to_np(v[0, h]), to_np(w), wl.blk_q, wl.blk_k, topk,
                                 mask=gidx, quant_group=32 if group32 else None)
            say(f"  topk {topk} head {h}: " + " ".join(f"{x:.3g}" for x in check_out(to_np(out[0, h]), r,
                                                                                       lin=to_np(ex["o_lin"][0, h]))))


def test_deterministic():
    wl = SMALL["grid"]
    q, k, v, w = (t.cuda() for t in synth.make(wl, 1))
    o1, e1 = run_gpu(q, k, v, w, wl, wl.topk)
    o2, e2 = run_gpu(q, k, v, w, wl, wl.topk)
    assert torch.equal(o1, o2)
    for name in e1:
        assert torch.equal(e1[name], e2[name]), name


def test_concurrent_streams():
    # the library keeps no state between calls: two forwards of different inputs, each with its own workspace, run
    # at once on two streams (default priority) and give the bits each gives alone
    wl = SMALL["ragged128"]
    cfg = sg.Config(wl.B, wl.H, wl.N, wl.D, wl.blk_q, wl.blk_k, wl.topk, wl.linear)
    ins = [[t.cuda() for t in synth.make(wl, seed)] for seed in (3, 4)]
    alone = [run_gpu(*x, wl, wl.topk)[0] for x in ins]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.empty(sg.workspace_bytes(cfg), dtype=torch.uint8, device="cuda") for _ in range(2)]
    outs = [torch.empty_like(ins[i][0]) for i in range(2)]
    torch.cuda.synchronize()
    for rep in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                sg.forward(*ins[i], topk=wl.topk, blk_q=wl.blk_q, out=outs[i], workspace=wss[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], alone[i]), f"stream {i}, repetition {rep}"


def test_stage_entry_points_agree_with_forward():
    wl = SMALL["ragged128"]
    q, k, v, w = (t.cuda() for t in synth.make(wl, 2))
    out, ex = run_gpu(q, k, v, w, wl, 3)
    qx, ws = sg.quantize(q, k, blk_q=wl.blk_q)
    idx = sg.select(qx["q_pool"], qx["k_pool"], N=wl.N, topk=3, blk_q=wl.blk_q, workspace=ws)
    torch.cuda.synchronize()
    for name in ("q_i8", "k_i8", "q_scale", "k_scale", "k_mean", "q_pool", "k_pool"):
        assert torch.equal(qx[name], ex[name]), name
    assert torch.equal(idx, ex["block_idx"][..., :3])


# ---------------------------------------------------------------------------------------------------------
# the real layer shapes, in the launch configuration the benchmark times, checked on sampled (b, h) heads
# and sampled query blocks (quantization and selection of a sampled head are checked in full)
# ---------------------------------------------------------------------------------------------------------
def sampled_case(cfg_id, heads, n_blocks_sample=6, seed=0, group32=False, norm=False):
    wl = synth.workload(cfg_id) if isinstance(cfg_id, int) else cfg_id
    say(f"full-size {wl.name} B{wl.B} H{wl.H} N{wl.N} topk {wl.topk}/{wl.n_kb}: generating")
    q, k, v, w = synth.make(wl, seed, device="cuda")
    nw = synth.make_norm_weights(wl.H, wl.D, seed, device="cuda") if norm else None
    torch.cuda.synchronize()
    say(f"full-size {wl.name}: forward (group32 {group32}, norm {norm})")
    out, ex = run_gpu(q, k, v, w, wl, wl.topk, linear=wl.linear, group32=group32,
                      norm=(nw[0], nw[1], synth.NORM_EPS) if norm else None)
    W = to_np(w)
    rng = np.random.default_rng(cfg_id if isinstance(cfg_id, int) else wl.N)
    flagged = 0
    for (b, h) in heads:
        Q, K, V = to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h])
        if norm:
            qh, eq = oracle_norm(q, b, nw[0])
            kh, ek = oracle_norm(k, b, nw[1])
            assert eq and ek
            Q, K = qh[h], kh[h]
            del qh, kh
            check_hat(ex, b, h, Q, "q_hat")
            check_hat(ex, b, h, K, "k_hat")
        gidx = ex["block_idx"][b, h].cpu().numpy()[:, :wl.topk]
        blocks = sorted(set([0, wl.n_qb - 1] + list(rng.choice(wl.n_qb, n_blocks_sample, replace=False))))
        say(f"  b{b} h{h}: oracle")
        r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, wl.topk, linear=wl.linear, mask=gidx, blocks=blocks,
                             quant_group=32 if group32 else None)
        assert r["exact_sum_ok"]
        check_quant(ex, r, b, h)
        sratio = check_scores(ex, r, b, h)
        flagged_h = check_mask(gidx, r, wl.topk)
        flagged += flagged_h
        rows = np.concatenate([np.arange(wl.N)[orc.block_rows(wl.N, wl.blk_q, I)] for I in blocks])
        lin = to_np(ex["o_lin"][b, h]) if wl.linear else None
        err, c = check_out(to_np(out[b, h]), r, rows=rows, lin=lin)
        say(f"  b{b} h{h}: {len(blocks)} query blocks, out max-abs {err:.2e} cos {c:.6f}, near-tie rows {flagged_h}"
            f", min gap {np.min(r['gap']):.2e}, score difference {sratio:.3f} of its bound")
    del q, k, v, out, ex
    torch.cuda.empty_cache()
    return flagged


def test_full_size_dense_480p():
    sampled_case(1, [(0, 0), (0, 11)])


def test_full_size_sla_480p():
    sampled_case(2, [(0, 0), (0, 7)])


def test_full_size_sla_720p_pair():
    sampled_case(3, [(0, 0), (1, 39)])


def test_full_size_sla_1080p_long():
    # the largest layer shape (N = 269280 tokens, 4208 key blocks, top-k 210), two heads sampled
    sampled_case(4, [(0, 0), (0, 39)])


def test_full_size_sla_720p_pair_group32():
    # the benchmarked layer with one INT8 scale per 32 tokens of Q and of K
    sampled_case(3, [(0, 0), (1, 39)], group32=True)


def test_full_size_sla_480p_qk_norm():
    # the 1.3B 480P layer with the RMSNorm of Q and K before the path
    sampled_case(2, [(0, 0), (0, 11)], norm=True)


def test_full_size_sla_720p_pair_qk_norm():
    # the benchmarked layer with the RMSNorm of Q and K before the path
    sampled_case(3, [(0, 0), (1, 39)], norm=True)


@pytest.mark.timeout(600)
def test_full_size_large_batch():
    # the 720P layer at batch 8 (B H N D = 8 40 75600 128): every activation tensor holds 3.1e9 elements (more than
    # 2^31), so any 32-bit element or byte offset would wrap; the first and the last head are checked
    wl = synth.custom(8, 40, 75600, grid=(21, 45, 80), structured=True, blk_q=128, topk_frac=0.1, name="720p-b8")
    assert wl.B * wl.H * wl.N * wl.D > 2 ** 31
    sampled_case(wl, [(0, 0), (7, 39)], n_blocks_sample=4)


def test_max_heads():
    # B * H = 65535, the largest head count (grid dimensions), 200 tokens per head with 2 of 4 key blocks selected
    # and the linear branch on; the first, a middle and the last head against the oracle
    wl = synth.custom(255, 257, 200, blk_q=128, topk_frac=0.5, name="max-heads")
    assert wl.B * wl.H == 65535 and wl.topk == 2
    q, k, v, w = synth.make(wl, 5, device="cuda")
    say(f"case {wl.name} B{wl.B} H{wl.H} N{wl.N}: forward")
    out, ex = run_gpu(q, k, v, w, wl, wl.topk)
    W = to_np(w)
    for (b, h) in [(0, 0), (127, 128), (254, 256)]:
        Q, K, V = to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h])
        gidx = ex["block_idx"][b, h].cpu().numpy()[:, :wl.topk]
        r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, wl.topk, linear=True)
        check_quant(ex, r, b, h)
        check_scores(ex, r, b, h)
        assert check_mask(gidx, r, wl.topk) == 0
        rg = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, wl.topk, linear=True, mask=gidx)
        err, c = check_out(to_np(out[b, h]), rg, lin=to_np(ex["o_lin"][b, h]))
        say(f"  b{b} h{h}: out max-abs {err:.2e} cos {c:.6f}")


@pytest.mark.timeout(600)
def test_full_size_max_key_blocks():
    # the largest key-block count the parameter checks accept (20480, N = 1310697 with a ragged last block),
    # 10% selected (2048-entry lists), linear branch on; the oracle ranks every query block's 20480 scores
    wl = synth.custom(1, 1, 20480 * 64 - 23, blk_q=128, topk_frac=0.1, name="max-key-blocks")
    assert wl.n_kb == 20480 and wl.topk == 2048
    sampled_case(wl, [(0, 0)], n_blocks_sample=3)


# ---------------------------------------------------------------------------------------------------------
# selection lists longer than the attention kernel keeps in LDS (1020 entries, 510 with 32-token groups): the
# kernel then reads block indices and key scales through scalar loads
# ---------------------------------------------------------------------------------------------------------
def test_long_list_dense_scalar_path():
    # dense top-k over 1021 key blocks, linear branch off
    wl = synth.custom(1, 1, 1021 * 64, blk_q=128, topk_frac=1.0, linear=False, name="dense-1021kb")
    assert wl.topk == 1021
    sampled_case(wl, [(0, 0)], n_blocks_sample=4)


def test_long_list_sparse_linear_scalar_path():
    # 1021 of 1100 key blocks selected (the ragged last key block holds 14 keys), linear branch on
    wl = synth.custom(1, 1, 70350, blk_q=128, topk_frac=1021 / 1100, name="sla-1021of1100")
    assert wl.topk == 1021 and wl.n_kb == 1100
    sampled_case(wl, [(0, 0)], n_blocks_sample=4)


def test_long_list_group32_scalar_path():
    # 32-token groups with 600 selected blocks (more than the 510 the LDS list holds in this mode)
    wl = synth.custom(1, 1, 40000, blk_q=128, topk_frac=600 / 625, name="sla-g32-600of625")
    assert wl.topk == 600 and wl.n_kb == 625
    sampled_case(wl, [(0, 0)], n_blocks_sample=4, group32=True)


# ---------------------------------------------------------------------------------------------------------
# top-k on more than 256 candidates: the histogram passes, exact ties (lower block index first) and the
# radix passes that take over when value-range passes stall, against the oracle's brute-force ranking on
# pooled means given directly (small integers and powers of two, so every score is exact on both sides)
# ---------------------------------------------------------------------------------------------------------
def select_case(qp, kp, topk, blk_q=128):
    n_kb = kp.shape[0]
    N = n_kb * 64
    assert qp.shape[0] == -(-N // blk_q)
    got = sg.select(torch.from_numpy(qp)[None, None].cuda(), torch.from_numpy(kp)[None, None].cuda(), N=N,
                    topk=topk, blk_q=blk_q)
    torch.cuda.synchronize()
    got = got.cpu().numpy()[0, 0]
    want, _ = orc.select_topk(orc.block_scores(qp, kp), topk)
    bad = [I for I in range(want.shape[0]) if not np.array_equal(got[I], want[I])]
    assert not bad, f"{len(bad)} rows differ, first {bad[:5]}: got {got[bad[0]][:12]} want {want[bad[0]][:12]}"
    return want


def test_select_all_scores_equal():
    # every key block has the same pooled mean: each row keeps blocks 0..k-1
    rng = np.random.default_rng(40)
    n_kb, D = 600, 128
    qp = rng.integers(-3, 4, size=(n_kb // 2, D)).astype(np.float64)
    kp = np.repeat(rng.integers(-3, 4, size=(1, D)).astype(np.float64), n_kb, axis=0)
    want = select_case(qp, kp, 60)
    assert (want == np.arange(60)).all()


@pytest.mark.parametrize("topk", [200, 400])
def test_select_two_score_values(topk):
    # key-block means take two values (300 blocks high, 700 low along channel 0); query rows of either sign, so
    # the k-th place falls inside a tier of 300 or 700 tied candidates
    rng = np.random.default_rng(41)
    n_kb, D = 1000, 128
    a = np.ones(n_kb)
    a[rng.permutation(n_kb)[:300]] = 2.0
    kp = np.zeros((n_kb, D))
    kp[:, 0] = a
    qp = np.zeros((n_kb // 2, D))
    qp[:, 0] = rng.choice([-3.0, -1.0, 1.0, 2.0], size=n_kb // 2)
    select_case(qp, kp, topk)


def test_select_scores_over_many_binades():
    # scores +-2^-e over 600 binades: equal-width value bins cut off only ~8 binades per pass, so the radix
    # passes must finish the selection
    rng = np.random.default_rng(42)
    n_kb, D = 600, 128
    kp = np.zeros((n_kb, D))
    kp[:, 0] = np.ldexp(1.0, -rng.permutation(n_kb))
    qp = np.zeros((n_kb // 2, D))
    qp[:, 0] = rng.choice([-1.0, 1.0], size=n_kb // 2)
    select_case(qp, kp, 300)
