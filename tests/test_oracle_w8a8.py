"""Pins of the W8A8 oracle to things other than itself (CPU only).

Each test checks the oracle against a fact the method or the mathematics fixes: lossless cases that reduce to
a plain integer or fp64 matrix product (numpy), IEEE fp32 division done by numpy, the quantizer's error bound,
saturation under clipping, and a hand-worked fixture under tests/golden/.
"""
import json
import os

import numpy as np
import pytest

from oracle import w8a8 as ow

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def exact_blocks(rng, R, C, exps):
    """Integers in [-127, 127] times 2^e of their 128x128 block, each block holding one +-127: the quantizer
    must give back the integers as codes and 2^e as the scale (absmax / 127 = 2^e exactly)."""
    ints = rng.integers(-127, 128, size=(R, C)).astype(np.int64)
    X = np.zeros((R, C), dtype=np.float64)
    for mb in range(ow.n_blocks(R)):
        r0, r1 = mb * 128, min(R, mb * 128 + 128)
        for kb in range(C // 128):
            ints[r0, kb * 128 + (mb + kb) % 128] = 127 if (mb + kb) % 2 else -127
            X[r0:r1, kb * 128:kb * 128 + 128] = np.ldexp(ints[r0:r1, kb * 128:kb * 128 + 128].astype(np.float64),
                                                         int(exps[mb, kb]))
    return ints, X


def test_quantizer_lossless_on_scaled_integers(rng):
    R, C = 300, 384  # ragged last row block (44 rows)
    exps = rng.integers(-6, 7, size=(ow.n_blocks(R), C // 128))
    ints, X = exact_blocks(rng, R, C, exps)
    codes, scales = ow.quantize_blocks(X)
    np.testing.assert_array_equal(codes.astype(np.int64), ints)
    np.testing.assert_array_equal(scales, np.ldexp(1.0, exps))


def test_quantizer_roundtrip_bound_and_ieee_fp32(rng):
    X = rng.standard_normal((200, 256)) * np.exp(rng.standard_normal((200, 1)))
    X = X.astype(np.float32).astype(np.float64)
    codes, scales = ow.quantize_blocks(X)
    deq = ow.dequantize_blocks(codes, scales)
    s_el = np.repeat(np.repeat(scales, 128, axis=0)[:200], 128, axis=1)
    assert np.all(np.abs(deq - X) <= s_el / 2 * (1 + 1e-6))
    # the codes are the round-half-even of the IEEE fp32 quotient, computed here by numpy's float32 division
    q = np.rint(X.astype(np.float32) / s_el.astype(np.float32))
    np.testing.assert_array_equal(codes, np.clip(q, -127, 127).astype(np.int8))
    # and the scale is the IEEE fp32 quotient absmax / 127
    amax = np.max(np.abs(X[:128, :128]))
    assert scales[0, 0] == float(np.float32(amax) / np.float32(127.0))


def test_round_half_even():
    X = np.zeros((1, 128))
    X[0, :6] = [127.0, 2.5, 3.5, -2.5, 126.5, -0.5]  # absmax 127: scale 1, quotients exact
    codes, scales = ow.quantize_blocks(X)
    assert scales[0, 0] == 1.0
    assert list(codes[0, :6]) == [127, 2, 4, -2, 126, 0]


def test_golden_clip_fixture():
    g = json.load(open(os.path.join(GOLDEN, "w8a8_clip_block.json")))
    X = np.zeros((1, 128))
    X[0, :len(g["x"])] = g["x"]
    codes, scales = ow.quantize_blocks(X, g["clip"])
    assert scales[0, 0] == float(g["scale_fp32"])
    assert list(codes[0, :len(g["x"])]) == g["codes"]
    assert not codes[0, len(g["x"]):].any()


def test_clipping_saturates_and_bounds_the_rest(rng):
    X = rng.standard_normal((128, 256))
    X[5, 7] = 40.0  # an outlier in block (0, 0)
    for alpha in (1.0, 0.5, 0.125):
        codes, scales = ow.quantize_blocks(X, alpha)
        for kb in range(2):
            blk = X[:, kb * 128:kb * 128 + 128]
            c = codes[:, kb * 128:kb * 128 + 128].astype(np.float64)
            s = scales[0, kb]
            t = float(np.float32(np.float32(alpha) * np.float32(np.max(np.abs(blk)))))
            assert s == float(np.float32(np.float32(t) / np.float32(127.0)))
            over = np.abs(blk) >= t
            assert np.all(np.abs(c[over]) == 127) and np.all(np.sign(c[over]) == np.sign(blk[over]))
            inside = np.abs(blk) < t * (126.5 / 127)
            assert np.all(np.abs(c[inside] * s - blk[inside]) <= s / 2 * (1 + 1e-6))


def test_zero_block():
    X = np.zeros((130, 256))
    X[:, 128:] = 1.0
    codes, scales = ow.quantize_blocks(X)
    assert scales[0, 0] == 0.0 and scales[1, 0] == 0.0 and not codes[:, :128].any()
    assert scales[0, 1] == float(np.float32(1.0) / np.float32(127.0)) and np.all(codes[:, 128:] == 127)


def test_gemm_equals_integer_matmul(rng):
    # scale 1 everywhere: the layer is the integer matrix product plus the bias
    M, N, K = 200, 256, 384
    ints_x, X = exact_blocks(rng, M, K, np.zeros((2, 3), dtype=int))
    ints_w, W = exact_blocks(rng, N, K, np.zeros((2, 3), dtype=int))
    b = rng.integers(-1000, 1000, size=N).astype(np.float64)
    Y, _, _ = ow.linear(X, W, b)
    np.testing.assert_array_equal(Y, (ints_x @ ints_w.T).astype(np.float64) + b[None, :])


def test_gemm_block_scales_lossless(rng):
    # a different power of two per block of X and of W: a scale taken from the wrong block changes the result
    M, N, K = 300, 384, 512
    ex = rng.integers(-3, 4, size=(ow.n_blocks(M), K // 128))
    ew = rng.integers(-3, 4, size=(N // 128, K // 128))
    _, X = exact_blocks(rng, M, K, ex)
    _, W = exact_blocks(rng, N, K, ew)
    Y, _, _ = ow.linear(X, W)
    np.testing.assert_array_equal(Y, X @ W.T)  # exact in fp64: integer multiples of 2^-6 below 2^40


def test_gemm_within_quantization_bound(rng):
    # |x^ w^ - x w| <= |x| e_w + |w| e_x + e_x e_w with e = s / 2 per element: summed, a closed-form bound
    M, N, K = 150, 256, 256
    X = rng.standard_normal((M, K)) * 3
    W = rng.standard_normal((N, K)) / 16
    b = rng.standard_normal(N)
    Y, (xq, xs), (wq, ws) = ow.linear(X, W, b)
    ref = X @ W.T + b[None, :]
    ex = np.repeat(np.repeat(xs, 128, axis=0)[:M], 128, axis=1) / 2
    ew = np.repeat(np.repeat(ws, 128, axis=0)[:N], 128, axis=1) / 2
    bound = np.abs(X) @ ew.T + ex @ np.abs(W).T + ex @ ew.T
    assert np.all(np.abs(Y - ref) <= bound * (1 + 1e-9) + 1e-12)
    assert np.max(np.abs(Y - ref)) > 0  # the bound is exercised, not trivially met


def test_abs_terms_bounds_and_matches_without_cancellation(rng):
    M, N, K = 130, 128, 256
    X = np.abs(rng.standard_normal((M, K)))
    W = np.abs(rng.standard_normal((N, K)))
    _, (xq, xs), (wq, ws) = ow.linear(X, W)
    A = ow.abs_terms(xq, xs, wq, ws)
    np.testing.assert_allclose(A, ow.block_gemm(xq, xs, wq, ws), rtol=1e-14)
    X2 = rng.standard_normal((M, K))
    _, (xq, xs), _ = ow.linear(X2, W)
    assert np.all(ow.abs_terms(xq, xs, wq, ws) >= np.abs(ow.block_gemm(xq, xs, wq, ws)) * (1 - 1e-14))


def test_rejects_bad_shapes_and_clip():
    with pytest.raises(ValueError):
        ow.quantize_blocks(np.ones((4, 100)))
    with pytest.raises(ValueError):
        ow.quantize_blocks(np.ones((4, 128)), 0.0)
    with pytest.raises(ValueError):
        ow.quantize_blocks(np.ones((4, 128)), 1.5)
