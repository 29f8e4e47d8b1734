"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch every one of them.

Each mutation replaces one oracle function with a subtly wrong version (a dropped term, a wrong sign, index or
constant, a transposed operand). The pins of test_oracle_pins must then fail somewhere.
"""
import math

import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import sagesla as orc

_orig = {name: getattr(orc, name) for name in orc.__all__}


def _phi_no_plus_one(x):
    x = np.asarray(x, np.float64)
    return np.where(x > 0, x, np.expm1(np.minimum(x, 0.0)))


def _quantize_div128(X, blk):
    codes, scales = _orig["quantize"](X * (127.0 / 128.0), blk)
    return codes, scales * (128.0 / 127.0)


def _quantize_floor(X, blk):
    X = np.asarray(X, np.float64)
    codes, scales = _orig["quantize"](X, blk)
    n = X.shape[0]
    for i, s in enumerate(scales):
        r = orc.block_rows(n, blk, i)
        if s:
            codes[r] = np.clip(np.floor((X[r] / s).astype(np.float32)), -127, 127).astype(np.int8)
    return codes, scales


def _select_ascending(scores, k):
    return _orig["select_topk"](-scores, k)


def _select_ties_high(scores, k):
    idx, gap = _orig["select_topk"](scores[:, ::-1], k)
    n = scores.shape[1]
    return np.sort(n - 1 - idx, axis=1), gap


def _linear_no_subtraction(Q, H, Z, idx, blk_q, **kw):
    empty = np.zeros((idx.shape[0], 0), dtype=np.int32)
    return _orig["linear_branch"](Q, H, Z, empty, blk_q, **kw)


def _linear_states_transposed(K, V, blk_k):
    H, Z = _orig["linear_states"](K, V, blk_k)
    return np.transpose(H, (0, 2, 1)).copy(), Z


def _kmean_first_block(K):
    return _orig["k_mean"](np.asarray(K)[:64])


def _sparse_no_scale(q_codes, q_scales, k_codes, k_scales, V, idx, blk_q, blk_k, sm_scale, **kw):
    return _orig["sparse_attention"](q_codes, q_scales, k_codes, k_scales, V, idx, blk_q, blk_k, 1.0, **kw)


def _sparse_drop_ragged_tail(q_codes, q_scales, k_codes, k_scales, V, idx, blk_q, blk_k, sm_scale, **kw):
    # forgets the last (ragged) key block's rows
    N = V.shape[0]
    nkb = orc.n_blocks(N, blk_k)
    idx2 = [np.array([J for J in row if J != nkb - 1] or [0]) for row in idx]
    return _orig["sparse_attention"](q_codes, q_scales, k_codes, k_scales, V, idx2, blk_q, blk_k, sm_scale, **kw)


def _sparse_ignore_groups(q_codes, q_scales, k_codes, k_scales, V, idx, blk_q, blk_k, sm_scale, blocks=None,
                          q_group=None, k_group=None):
    # indexes finer scales as if there were one per block
    return _orig["sparse_attention"](q_codes, q_scales, k_codes, k_scales, V, idx, blk_q, blk_k, sm_scale,
                                     blocks=blocks)


def _pool_sum(X, blk):
    return _orig["pool"](X, blk) * blk


def _project_transposed(O_l, W_p):
    return _orig["project"](O_l, np.asarray(W_p).T)


def _rmsnorm_per_head(X, gamma, eps):
    # normalizes each head's D channels alone instead of all H*D channels of the token
    X = np.asarray(X, np.float64)
    H, N, D = X.shape
    g = np.asarray(gamma, np.float64).reshape(H, D)
    outs, rs = [], []
    for h in range(H):
        y, r, ex = _orig["qk_rmsnorm"](X[h:h + 1], g[h], eps)
        outs.append(y[0])
        rs.append(r)
    return np.stack(outs), rs[0], np.zeros(N, dtype=bool)


def _rmsnorm_no_weight(X, gamma, eps):
    return _orig["qk_rmsnorm"](X, np.ones_like(np.asarray(gamma, np.float64)), eps)


def _rmsnorm_sum_not_mean(X, gamma, eps):
    # divides by the root of the sum of squares instead of their mean
    X = np.asarray(X, np.float64)
    H, N, D = X.shape
    S = (X * X).sum(axis=(0, 2))
    r = (1.0 / np.sqrt(S + float(np.float32(eps)))).astype(np.float32).astype(np.float64)
    n = orc.bf16_round(X * r[None, :, None])
    return orc.bf16_round(n * np.asarray(gamma, np.float64).reshape(H, 1, D)), r, np.zeros(N, dtype=bool)


def _bf16_ties_away(x):
    # round half away from zero instead of to even
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x8000) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _bf16_truncate(x):
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    return (u & 0xFFFF0000).astype(np.uint32).view(np.float32).astype(np.float64)


def _bf16_bias_off_by_one(x):
    # 0x8000 instead of 0x7FFF in the rounding constant: ties of even kept parts round up
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x8000 + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


MUTATIONS = {
    "bf16_ties_away": ("bf16_round", _bf16_ties_away),
    "bf16_truncate": ("bf16_round", _bf16_truncate),
    "bf16_bias_off_by_one": ("bf16_round", _bf16_bias_off_by_one),
    "rmsnorm_per_head": ("qk_rmsnorm", _rmsnorm_per_head),
    "rmsnorm_no_weight": ("qk_rmsnorm", _rmsnorm_no_weight),
    "rmsnorm_sum_not_mean": ("qk_rmsnorm", _rmsnorm_sum_not_mean),
    "phi_no_plus_one": ("phi", _phi_no_plus_one),
    "quantize_div128": ("quantize", _quantize_div128),
    "quantize_floor": ("quantize", _quantize_floor),
    "select_ascending": ("select_topk", _select_ascending),
    "select_ties_high": ("select_topk", _select_ties_high),
    "linear_no_subtraction": ("linear_branch", _linear_no_subtraction),
    "linear_states_transposed": ("linear_states", _linear_states_transposed),
    "kmean_first_block": ("k_mean", _kmean_first_block),
    "sparse_no_scale": ("sparse_attention", _sparse_no_scale),
    "sparse_drop_ragged_tail": ("sparse_attention", _sparse_drop_ragged_tail),
    "sparse_ignore_groups": ("sparse_attention", _sparse_ignore_groups),
    "project_transposed": ("project", _project_transposed),
    "pool_sum": ("pool", _pool_sum),
}


def _run_pins():
    rng = lambda: np.random.default_rng(1234)
    checks = [
        lambda: pins.test_dense_equivalence_unsmoothed(pins.SMALL[1]),
        lambda: pins.test_dense_equivalence_quantized(),
        lambda: pins.test_smoothing_invariance(),
        lambda: pins.test_kmean_exact_sum(),
        lambda: pins.test_quant_roundtrip_and_ieee_fp32(rng()),
        lambda: pins.test_golden_quant_fixture(),
        lambda: pins.test_select_bruteforce(rng()),
        lambda: pins.test_select_constant_keys_and_full(),
        lambda: pins.test_block_score_is_mean_token_score(),
        lambda: pins.test_sparse_bruteforce(rng()),
        lambda: pins.test_sparse_bruteforce_groups(rng()),
        lambda: pins.test_dense_equivalence_quantized_groups(pins.SMALL[1]),
        lambda: pins.test_linear_closed_form_all_marginal(pins.SMALL[0]),
        lambda: pins.test_linear_bruteforce_marginal_keys(rng()),
        lambda: pins.test_phi_matches_library(rng()),
        lambda: pins.test_combine_special_cases(),
        lambda: pins.test_rmsnorm_matches_library(),
        lambda: pins.test_rmsnorm_unit_rms_with_unit_weight(),
        lambda: pins.test_bf16_round_matches_library_and_ties(),
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failed += 1
    return failed


def test_pins_pass_unmutated():
    assert _run_pins() == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(orc, attr, fn)
    assert _run_pins() > 0, f"planted mistake {name} passed every pin"
