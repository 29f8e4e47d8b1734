"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test checks the oracle against a fact the method or the mathematics fixes: a special case that reduces
to a library routine (dense softmax attention, elu), a closed form, an invariance, brute force on tiny inputs,
IEEE fp32 arithmetic done by numpy, or a hand-worked fixture under tests/golden/.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import sagesla as orc
from conftest import to_np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def head(wl, seed=0, b=0, h=0):
    q, k, v, w = synth.make(wl, seed)
    return to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h]), to_np(w)


def sdpa64(Q, K, V, scale):
    """Library dense attention (torch, fp64, CPU)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V), scale=scale)[0, 0].numpy()


SMALL = [
    synth.custom(1, 1, 512, blk_q=128, blk_k=64),
    synth.custom(1, 1, 1000, blk_q=128, blk_k=64),  # ragged: q tail 104, k tail 40
    synth.custom(1, 1, 330, blk_q=64, blk_k=64),  # ragged: tails 10
    synth.custom(1, 1, 6 * 7 * 8, grid=(6, 7, 8), structured=True, blk_q=64, blk_k=64),
]


# ---------------------------------------------------------------------------------------------------------
# dense equivalence: top-k 100 %, quantization off -> textbook softmax attention
# ---------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"N{w.N}-bq{w.blk_q}")
def test_dense_equivalence_unsmoothed(wl):
    Q, K, V, W = head(wl)
    r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, wl.n_kb, linear=False, smooth_k=False, quant=False)
    ref = sdpa64(Q, K, V, 1 / math.sqrt(wl.D))
    np.testing.assert_allclose(r["out"], ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"N{w.N}-bq{w.blk_q}")
def test_dense_equivalence_smoothed(wl):
    # smoothing only adds the fp32 rounding of k' = K - mu (relative 2^-24), nothing else
    Q, K, V, W = head(wl)
    r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, wl.n_kb, linear=False, smooth_k=True, quant=False)
    ref = sdpa64(Q, K, V, 1 / math.sqrt(wl.D))
    np.testing.assert_allclose(r["out"], ref, atol=2e-5, rtol=0)


def test_dense_equivalence_quantized():
    # top-k 100 % with quantization on == dense attention on the dequantized Q and smoothed K
    wl = SMALL[1]
    Q, K, V, W = head(wl)
    r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, wl.n_kb, linear=False)
    Qd = r["q_codes"].astype(np.float64) * np.repeat(r["q_scales"], wl.blk_q)[: wl.N, None]
    Kd = r["k_codes"].astype(np.float64) * np.repeat(r["k_scales"], wl.blk_k)[: wl.N, None]
    ref = sdpa64(Qd, Kd, V, 1 / math.sqrt(wl.D))
    np.testing.assert_allclose(r["out"], ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("wl", SMALL[:3], ids=lambda w: f"N{w.N}-bq{w.blk_q}")
def test_dense_equivalence_quantized_groups(wl):
    # thread-level granularity ([TD-news] §三(一) item 2): one scale per 32 tokens of Q and of K. Top-k 100 %
    # then equals dense attention on Q and smoothed K dequantized group by group (ragged last groups included)
    Q, K, V, W = head(wl)
    r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, wl.n_kb, linear=False, quant_group=32)
    ng = -(-wl.N // 32)
    assert len(r["q_scales"]) == ng and len(r["k_scales"]) == ng
    for codes, scales in ((r["q_codes"], r["q_scales"]), (r["k_codes"], r["k_scales"])):
        for g in range(ng):  # each group's absmax element maps to +-127
            if scales[g] > 0:
                assert np.max(np.abs(codes[32 * g: 32 * g + 32].astype(int))) == 127
    Qd = r["q_codes"].astype(np.float64) * np.repeat(r["q_scales"], 32)[: wl.N, None]
    Kd = r["k_codes"].astype(np.float64) * np.repeat(r["k_scales"], 32)[: wl.N, None]
    ref = sdpa64(Qd, Kd, V, 1 / math.sqrt(wl.D))
    np.testing.assert_allclose(r["out"], ref, atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------------------------------------
# K-mean smoothing
# ---------------------------------------------------------------------------------------------------------
def test_smoothing_invariance():
    # subtracting one vector from every key leaves each softmax row unchanged; here only the fp32 rounding of
    # k' differs, so the outputs agree to that rounding, and far below what a wrong mean would give
    wl = SMALL[1]
    Q, K, V, W = head(wl)
    a = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, 3, linear=False, smooth_k=True, quant=False)
    b = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, 3, linear=False, smooth_k=False, quant=False,
                         mask=a["idx"])
    np.testing.assert_allclose(a["out"], b["out"], atol=2e-5, rtol=0)
    # the selection is invariant too: logits of a row shift by qbar_I . mu / sqrt(D)
    assert np.array_equal(a["idx"], b["idx"])
    # and the smoothing matters for the quantization: the bias dominates raw K's absmax
    assert np.mean(np.abs(a["mu"])) > 0.5


def test_kmean_exact_sum():
    Q, K, V, W = head(SMALL[1])
    assert orc.exact_sum_ok(K)
    mu = orc.k_mean(K)
    for c in range(K.shape[1]):
        ref = float(np.float32(math.fsum(K[:, c]) / K.shape[0]))
        assert mu[c] == ref


def test_exact_sum_precondition_detects_failure():
    x = np.array([[2.0 ** 60], [2.0 ** -10]])
    assert not orc.exact_sum_ok(x)
    assert orc.exact_sum_ok(np.array([[1.0], [2.0 ** -10]]))
    # granularity is the value's lowest set bit, not its precision: 3 * 2^-40 needs 2^-40, 1.5 needs 2^-1
    assert not orc.exact_sum_ok(np.array([[2.0 ** 13], [3 * 2.0 ** -40]]))
    assert orc.exact_sum_ok(np.array([[2.0 ** 13], [3 * 2.0 ** -38]]))
    # when the precondition holds the fp64 sum equals math.fsum in any order
    rng = np.random.default_rng(0)
    col = (rng.standard_normal(20000) * 2 + 1).astype(np.float32).astype(np.float64)
    import torch
    col = torch.from_numpy(col).to(torch.bfloat16).double().numpy()
    assert orc.exact_sum_ok(col[:, None])
    assert float(np.sum(col)) == math.fsum(col) == float(np.sum(col[::-1])) == float(np.sum(np.sort(col)))


# ---------------------------------------------------------------------------------------------------------
# quantization
# ---------------------------------------------------------------------------------------------------------
def test_quant_roundtrip_and_ieee_fp32(rng):
    X = rng.standard_normal((300, 128)).astype(np.float32).astype(np.float64) * 3.0
    X[130:140] *= 50.0  # an outlier band inside block 1
    codes, scales = orc.quantize(X, 64)
    for i in range(orc.n_blocks(300, 64)):
        rows = orc.block_rows(300, 64, i)
        xb, cb, s = X[rows], codes[rows], scales[i]
        a = np.max(np.abs(xb))
        # scale is the fp32 quotient absmax/127 computed in IEEE fp32 by numpy
        assert s == float(np.float32(a) / np.float32(127.0))
        # codes == round-half-even of numpy's IEEE fp32 quotient, clamped
        ref = np.clip(np.rint(xb.astype(np.float32) / np.float32(s)), -127, 127)
        assert np.array_equal(cb.astype(np.float64), ref.astype(np.float64))
        # round trip within half a step (the fp32 quotient adds at most 127 * 2^-24 of a step)
        err = np.abs(xb - cb * s)
        assert np.all(err <= s / 2 * (1 + 2.0 ** -16))
        assert np.count_nonzero(err > s / 2) <= 2
        # the absmax element maps to +-127
        j = np.unravel_index(np.argmax(np.abs(xb)), xb.shape)
        assert abs(int(cb[j])) == 127


def test_quant_zero_block_and_half_even():
    X = np.zeros((128, 4))
    X[64:, 0] = 127.0  # block 1: absmax 127 -> scale exactly 1
    X[64, 1:4] = [0.5, 1.5, -2.5]  # exact halves round to even
    codes, scales = orc.quantize(X, 64)
    assert scales[0] == 0.0 and not codes[:64].any()
    assert scales[1] == 1.0
    assert list(codes[64, :4]) == [127, 0, 2, -2]


def test_golden_quant_fixture():
    with open(os.path.join(GOLDEN, "quant_block.json")) as f:
        g = json.load(f)
    X = np.array(g["x"], dtype=np.float64)[:, None]
    codes, scales = orc.quantize(X, len(g["x"]))
    assert float(scales[0]) == float(np.float32(g["scale_fp32"]))
    assert [int(c) for c in codes[:, 0]] == g["codes"]


# ---------------------------------------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------------------------------------
def test_select_bruteforce(rng):
    for trial in range(20):
        nq, nk = rng.integers(1, 9), rng.integers(1, 25)
        s = np.round(rng.standard_normal((nq, nk)), 1)  # coarse values: many exact ties
        k = int(rng.integers(0, nk + 1))
        idx, gap = orc.select_topk(s, k)
        for I in range(nq):
            order = sorted(range(nk), key=lambda J: (-s[I, J], J))
            assert list(idx[I]) == sorted(order[:k])
            if 0 < k < nk:
                assert gap[I] == s[I, order[k - 1]] - s[I, order[k]]


def test_select_constant_keys_and_full():
    wl = SMALL[0]
    Q, K, V, W = head(wl)
    Kc = np.ones_like(K) * 0.75  # every smoothed key is 0 -> all scores 0 -> ties -> lowest indices
    r = orc.forward_head(Q, Kc, V, W, wl.blk_q, wl.blk_k, 3)
    assert np.array_equal(r["idx"], np.tile(np.arange(3), (wl.n_qb, 1)))
    assert not r["k_codes"].any() and not r["k_scales"].any()
    r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, wl.n_kb)
    assert np.array_equal(r["idx"], np.tile(np.arange(wl.n_kb), (wl.n_qb, 1)))


def test_block_score_is_mean_token_score():
    # by linearity, qbar_I . kbar_J equals the average over the valid keys j of block J (and the valid queries
    # i of block I) of q_i . k'_j -- including the ragged last blocks
    wl = SMALL[1]
    Q, K, V, W = head(wl)
    r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, 2, linear=False)
    Kp = K - r["mu"][None, :]
    tok = Q @ Kp.T / math.sqrt(wl.D)
    for I in (0, wl.n_qb - 1):
        for J in (0, 3, wl.n_kb - 1):
            ref = tok[I * wl.blk_q:(I + 1) * wl.blk_q, J * wl.blk_k:(J + 1) * wl.blk_k].mean()
            assert abs(r["scores"][I, J] - ref) < 1e-5


def test_topk_count():
    assert [orc.topk_count(w.topk_frac, w.n_kb) for w in synth.WORKLOADS.values()] == [4, 512, 51, 118, 210]
    assert orc.topk_count(0.001, 10) == 1


def test_selection_prefers_local_blocks_on_structured_input():
    # a shared smooth field makes neighbouring blocks the most similar: the diagonal block is kept
    wl = synth.custom(1, 1, 8 * 16 * 16, grid=(8, 16, 16), structured=True, blk_q=64, blk_k=64)
    Q, K, V, W = head(wl)
    r = orc.forward_head(Q, K, V, W, 64, 64, 4, linear=False)
    assert np.mean([I in r["idx"][I] for I in range(wl.n_qb)]) > 0.9


# ---------------------------------------------------------------------------------------------------------
# sparse attention
# ---------------------------------------------------------------------------------------------------------
def test_sparse_bruteforce(rng):
    N, D, bq, bk = 150, 16, 32, 16
    Q = rng.standard_normal((N, D))
    K = rng.standard_normal((N, D)) + 1.0
    V = rng.standard_normal((N, D))
    qc, qs = orc.quantize(Q, bq)
    kc, ks = orc.quantize(K, bk)
    nqb, nkb = orc.n_blocks(N, bq), orc.n_blocks(N, bk)
    idx = np.stack([np.sort(rng.choice(nkb, 3, replace=False)) for _ in range(nqb)])
    out = orc.sparse_attention(qc, qs, kc, ks, V, idx, bq, bk, 0.3)
    for i in range(N):
        I = i // bq
        zs, vs = [], []
        for J in idx[I]:
            for j in range(J * bk, min(N, (J + 1) * bk)):
                dot = sum(int(qc[i, c]) * int(kc[j, c]) for c in range(D))
                zs.append(dot * qs[I] * ks[J] * 0.3)
                vs.append(V[j])
        m = max(zs)
        w = [math.exp(z - m) for z in zs]
        ref = sum(wi * vi for wi, vi in zip(w, vs)) / sum(w)
        np.testing.assert_allclose(out[i], ref, atol=1e-12, rtol=0)


def test_sparse_bruteforce_groups(rng):
    # one scale per 16 rows of Q and per 16 keys, groups 2^g apart in magnitude so a scale taken from the wrong
    # group shows; blocks of 48 queries / 32 keys, ragged tails
    N, D, bq, bk, grp = 150, 16, 48, 32, 16
    mag = np.repeat(2.0 ** (np.arange(-(-N // grp)) % 5), grp)[:N, None]
    Q = rng.standard_normal((N, D)) * mag
    K = (rng.standard_normal((N, D)) + 1.0) * mag[::-1]
    V = rng.standard_normal((N, D))
    qc, qs = orc.quantize(Q, grp)
    kc, ks = orc.quantize(K, grp)
    nqb, nkb = orc.n_blocks(N, bq), orc.n_blocks(N, bk)
    idx = np.stack([np.sort(rng.choice(nkb, 2, replace=False)) for _ in range(nqb)])
    out = orc.sparse_attention(qc, qs, kc, ks, V, idx, bq, bk, 0.05, q_group=grp, k_group=grp)
    for i in range(N):
        zs, vs = [], []
        for J in idx[i // bq]:
            for j in range(J * bk, min(N, (J + 1) * bk)):
                dot = sum(int(qc[i, c]) * int(kc[j, c]) for c in range(D))
                zs.append(dot * qs[i // grp] * ks[j // grp] * 0.05)
                vs.append(V[j])
        m = max(zs)
        w = [math.exp(z - m) for z in zs]
        ref = sum(wi * vi for wi, vi in zip(w, vs)) / sum(w)
        np.testing.assert_allclose(out[i], ref, atol=1e-12, rtol=0)


def test_sparse_block_order_invariance(rng):
    wl = SMALL[1]
    Q, K, V, W = head(wl)
    r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, 5, linear=False)
    perm = np.stack([rng.permutation(row) for row in r["idx"]])
    o2 = orc.sparse_attention(r["q_codes"], r["q_scales"], r["k_codes"], r["k_scales"], V, perm,
                              wl.blk_q, wl.blk_k, 1 / math.sqrt(wl.D))
    np.testing.assert_allclose(o2, r["o_s"], atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------------------------------------
# linear branch
# ---------------------------------------------------------------------------------------------------------
def _phi_lib(x):
    return torch.nn.functional.elu(torch.from_numpy(np.asarray(x, np.float64))).numpy() + 1.0


@pytest.mark.parametrize("wl", SMALL[:3], ids=lambda w: f"N{w.N}-bq{w.blk_q}")
def test_linear_closed_form_all_marginal(wl):
    # no critical block: O_l = phi(Q)(phi(K)^T V) / phi(Q).sum(phi(K)), the plain linear-attention closed form
    Q, K, V, W = head(wl)
    r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, 0)
    PQ, PK = _phi_lib(Q), _phi_lib(K)
    ref = (PQ @ (PK.T @ V)) / (PQ @ PK.sum(axis=0))[:, None]
    np.testing.assert_allclose(r["o_l"], ref, rtol=1e-11, atol=1e-13)
    assert not r["o_s"].any()
    np.testing.assert_allclose(r["out"], ref @ W, rtol=1e-10, atol=1e-12)


def test_linear_bruteforce_marginal_keys(rng):
    N, D, bq, bk = 100, 8, 16, 8
    Q = rng.standard_normal((N, D))
    K = rng.standard_normal((N, D)) * 2
    V = rng.standard_normal((N, D))
    nqb, nkb = orc.n_blocks(N, bq), orc.n_blocks(N, bk)
    idx = np.stack([np.sort(rng.choice(nkb, 4, replace=False)) for _ in range(nqb)])
    H, Z = orc.linear_states(K, V, bk)
    out = orc.linear_branch(Q, H, Z, idx, bq)
    f = lambda x: x + 1 if x > 0 else math.exp(x)
    for i in range(N):
        crit = set(int(J) for J in idx[i // bq])
        num = np.zeros(D)
        den = 0.0
        for j in range(N):
            if j // bk in crit:
                continue
            w = sum(f(Q[i, c]) * f(K[j, c]) for c in range(D))
            num += w * V[j]
            den += w
        np.testing.assert_allclose(out[i], num / den, rtol=1e-10, atol=1e-12)
        # convex combination of the remaining value rows
        marg = [j for j in range(N) if j // bk not in crit]
        assert np.all(out[i] <= V[marg].max(axis=0) + 1e-12) and np.all(out[i] >= V[marg].min(axis=0) - 1e-12)


def test_linear_zero_when_all_critical():
    wl = SMALL[2]
    Q, K, V, W = head(wl)
    r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, wl.n_kb)
    assert not r["o_l"].any()


def test_phi_matches_library(rng):
    x = rng.standard_normal(1000) * 4
    np.testing.assert_allclose(orc.phi(x), _phi_lib(x), rtol=1e-11, atol=0)  # torch uses expm1(x)+1


# ---------------------------------------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------------------------------------
def test_combine_special_cases():
    wl = SMALL[1]
    Q, K, V, W = head(wl)
    r = orc.forward_head(Q, K, V, np.zeros_like(W), wl.blk_q, wl.blk_k, 4)
    assert np.array_equal(r["out"], r["o_s"])
    r = orc.forward_head(Q, K, np.zeros_like(V), W, wl.blk_q, wl.blk_k, 4)
    assert not r["out"].any()
    r = orc.forward_head(Q, K, V, np.eye(wl.D), wl.blk_q, wl.blk_k, 4)
    np.testing.assert_allclose(r["out"], r["o_s"] + r["o_l"], atol=1e-15, rtol=0)


# ---------------------------------------------------------------------------------------------------------
# RMSNorm of Q and K over all heads of a token (the optional step before the path)
# ---------------------------------------------------------------------------------------------------------
def test_bf16_round_matches_library_and_ties():
    # bf16 round-to-nearest-even of exact fp32 values, against torch's fp32 -> bf16 conversion (RNE) on random
    # values over a wide exponent range, and against hand-worked exact ties: a value halfway between two bf16
    # neighbours goes to the one whose last kept mantissa bit is 0, for either sign
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(200000) * 2.0 ** rng.integers(-40, 40, size=200000)).astype(np.float32)
    # append patterns whose dropped half is exactly 0x8000 (ties), 0x7FFF and 0x8001 (just below / above a tie)
    expo = rng.integers(1, 254, size=4000, dtype=np.uint32)  # finite, normal
    base = (expo << 23) | (rng.integers(0, 1 << 7, size=4000, dtype=np.uint32) << 16)
    u = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001, (base | 0x8000) | 0x80000000])
    x = np.concatenate([x, u.view(np.float32)]).astype(np.float64)
    got = orc.bf16_round(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)
    # hand-worked: ulp of bf16 on [1, 2) is 2^-7
    cases = [
        (1 + 2.0 ** -8, 1.0),                      # tie, kept bit even (1.0000000) -> stays
        (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),        # tie between 1+2^-7 (odd) and 1+2^-6 (even) -> up
        (-(1 + 2.0 ** -8), -1.0),                  # negative tie, even -> magnitude stays
        (-(1 + 3 * 2.0 ** -8), -(1 + 2.0 ** -6)),  # negative tie, odd -> magnitude up
        (1 + 2.0 ** -8 + 2.0 ** -23, 1 + 2.0 ** -7),  # just above a tie -> up
        (1 + 3 * 2.0 ** -8 - 2.0 ** -23, 1 + 2.0 ** -7),  # just below a tie -> down
        (255.5, 256.0),                            # tie at ulp 1: 255 odd -> 256
        (254.5, 254.0),                            # ulp 1 below 256: 254 even -> stays
        (2.0 ** -130 * 1.5, 2.0 ** -130 * 1.5),    # fp32 subnormal with few bits: exact in bf16
    ]
    for v, want in cases:
        assert orc.bf16_round(np.array([v]))[0] == want, (v, want)


def _norm_inputs(H=3, N=50, D=128, seed=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((H, N, D)) * np.exp(rng.standard_normal((1, N, 1)))
    X = orc.bf16_round(X)
    gamma = orc.bf16_round(1 + 0.1 * rng.standard_normal(H * D))
    return X, gamma


def test_rmsnorm_matches_library():
    # torch's fp64 rms_norm over the H*D channels of each token, weight applied: the oracle differs only by its
    # two bf16 roundings (relative 2^-8 each at most) and r's fp32 rounding (2^-24): y = x r g (1+d1)(1+d2)(1+d3)
    X, gamma = _norm_inputs()
    H, N, D = X.shape
    Y, r, amb = orc.qk_rmsnorm(X, gamma, 1e-6)
    assert not amb.any()
    t = torch.from_numpy(X.transpose(1, 0, 2).reshape(N, H * D))
    ref = torch.nn.functional.rms_norm(t, (H * D,), torch.from_numpy(gamma), eps=float(np.float32(1e-6)))
    ref = ref.numpy().reshape(N, H, D).transpose(1, 0, 2)
    np.testing.assert_allclose(Y, ref, rtol=2.0 ** -7 + 2.0 ** -15, atol=0)
    assert np.max(np.abs(Y / ref - 1)) > 2.0 ** -9  # both roundings are really there
    # r itself: the fp32 rounding of the exact reciprocal root
    np.testing.assert_allclose(r, 1 / np.sqrt((X ** 2).mean(axis=(0, 2)) + float(np.float32(1e-6))), rtol=2.0 ** -24)


def test_rmsnorm_sum_of_squares_is_exact():
    # the double-double sum against Python's exactly rounded math.fsum, on values spanning 2^-60 .. 2^20
    rng = np.random.default_rng(9)
    v = orc.bf16_round(rng.standard_normal((3000, 7)) * 2.0 ** rng.integers(-30, 10, size=(3000, 7)))
    sq = v * v
    S = orc._sum_squares(sq)
    assert all(S[j] == math.fsum(sq[:, j]) for j in range(7))


def test_rmsnorm_scale_invariance_and_zero_token():
    X, gamma = _norm_inputs(seed=1)
    X[:, 7] = 0.0
    Y, r, _ = orc.qk_rmsnorm(X, gamma, 0.0 + 1e-30)  # eps far below every mean square
    X2 = X.copy()
    X2[:, 3] *= 2.0 ** 5
    X2[:, 4] *= 2.0 ** -7
    Y2, r2, _ = orc.qk_rmsnorm(X2, gamma, 1e-30)
    np.testing.assert_array_equal(Y2[:, 3], Y[:, 3])
    np.testing.assert_array_equal(Y2[:, 4], Y[:, 4])
    assert r2[3] == r[3] * 2.0 ** -5 and r2[4] == r[4] * 2.0 ** 7
    assert not Y[:, 7].any()


def test_rmsnorm_unit_rms_with_unit_weight():
    X, _ = _norm_inputs(seed=2)
    Y, _, _ = orc.qk_rmsnorm(X, np.ones(X.shape[0] * X.shape[2]), 1e-6)
    ms = (Y ** 2).mean(axis=(0, 2))
    np.testing.assert_allclose(ms, 1.0, rtol=2.0 ** -7)


def test_forward_with_norm_equals_forward_on_normalized_inputs():
    wl = SMALL[1]
    q, k, v, w = synth.make(synth.custom(1, 2, 1000, blk_q=128, blk_k=64), 0)
    gq, gk = synth.make_norm_weights(2, 128, 0)
    Q, K, V, W = to_np(q), to_np(k), to_np(v), to_np(w)
    res = orc.forward(Q, K, V, W, 128, 64, 3, qk_norm=(to_np(gq), to_np(gk), synth.NORM_EPS))
    qh = orc.qk_rmsnorm(Q[0], to_np(gq), synth.NORM_EPS)[0]
    kh = orc.qk_rmsnorm(K[0], to_np(gk), synth.NORM_EPS)[0]
    for h in range(2):
        r = orc.forward_head(qh[h], kh[h], V[0, h], W, 128, 64, 3)
        np.testing.assert_array_equal(res[0][h]["out"], r["out"])
        np.testing.assert_array_equal(res[0][h]["q_hat"], qh[h])
    del wl
