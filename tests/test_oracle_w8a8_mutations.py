"""Plant plausible mistakes in the W8A8 oracle (on the CPU) and check that its pins catch every one of them."""
import numpy as np
import pytest

import test_oracle_w8a8 as pins
from oracle import w8a8 as ow

_orig = {name: getattr(ow, name) for name in ("quantize_blocks", "block_gemm")}


def _quant_div128(X, clip=1.0):
    codes, scales = _orig["quantize_blocks"](np.asarray(X, np.float64) * (127.0 / 128.0), clip)
    return codes, scales * (128.0 / 127.0)


def _quant_floor(X, clip=1.0):
    X = np.asarray(X, np.float64)
    codes, scales = _orig["quantize_blocks"](X, clip)
    for mb in range(scales.shape[0]):
        for kb in range(scales.shape[1]):
            s = scales[mb, kb]
            if s:
                blk = X[mb * 128:mb * 128 + 128, kb * 128:kb * 128 + 128]
                codes[mb * 128:mb * 128 + 128, kb * 128:kb * 128 + 128] = np.clip(
                    np.floor((blk / s).astype(np.float32)), -127, 127).astype(np.int8)
    return codes, scales


def _quant_ignore_clip(X, clip=1.0):
    return _orig["quantize_blocks"](X, 1.0)


def _quant_clip_no_saturation(X, clip=1.0):
    # scales from the clipped threshold but codes wrapped to int8 instead of clamped
    X = np.asarray(X, np.float64)
    codes, scales = _orig["quantize_blocks"](X, clip)
    for mb in range(scales.shape[0]):
        for kb in range(scales.shape[1]):
            s = scales[mb, kb]
            if s:
                blk = X[mb * 128:mb * 128 + 128, kb * 128:kb * 128 + 128]
                q = np.rint((blk / s).astype(np.float32)).astype(np.int64)
                codes[mb * 128:mb * 128 + 128, kb * 128:kb * 128 + 128] = ((q + 128) % 256 - 128).astype(np.int8)
    return codes, scales


def _gemm_weight_scale_transposed(xq, xs, wq, ws, bias=None):
    ws = np.asarray(ws)
    if ws.shape[0] == ws.shape[1]:
        ws = ws.T
    else:  # use the scale of the next k-block
        ws = np.roll(ws, 1, axis=1)
    return _orig["block_gemm"](xq, xs, wq, ws, bias)


def _gemm_act_scale_first_block(xq, xs, wq, ws, bias=None):
    xs = np.repeat(np.asarray(xs)[:1], np.asarray(xs).shape[0], axis=0)
    return _orig["block_gemm"](xq, xs, wq, ws, bias)


def _gemm_drop_bias(xq, xs, wq, ws, bias=None):
    return _orig["block_gemm"](xq, xs, wq, ws, None)


def _gemm_codes_as_uint8(xq, xs, wq, ws, bias=None):
    return _orig["block_gemm"](np.asarray(xq).view(np.uint8), xs, wq, ws, bias)


MUTATIONS = {
    "quant_div128": ("quantize_blocks", _quant_div128),
    "quant_floor": ("quantize_blocks", _quant_floor),
    "quant_ignore_clip": ("quantize_blocks", _quant_ignore_clip),
    "quant_clip_wraps": ("quantize_blocks", _quant_clip_no_saturation),
    "gemm_weight_scale_transposed": ("block_gemm", _gemm_weight_scale_transposed),
    "gemm_act_scale_first_block": ("block_gemm", _gemm_act_scale_first_block),
    "gemm_drop_bias": ("block_gemm", _gemm_drop_bias),
    "gemm_codes_as_uint8": ("block_gemm", _gemm_codes_as_uint8),
}


def _run_pins():
    rng = lambda: np.random.default_rng(1234)
    checks = [
        lambda: pins.test_quantizer_lossless_on_scaled_integers(rng()),
        lambda: pins.test_quantizer_roundtrip_bound_and_ieee_fp32(rng()),
        lambda: pins.test_round_half_even(),
        lambda: pins.test_golden_clip_fixture(),
        lambda: pins.test_clipping_saturates_and_bounds_the_rest(rng()),
        lambda: pins.test_zero_block(),
        lambda: pins.test_gemm_equals_integer_matmul(rng()),
        lambda: pins.test_gemm_block_scales_lossless(rng()),
        lambda: pins.test_gemm_within_quantization_bound(rng()),
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
    monkeypatch.setattr(ow, attr, fn)
    assert _run_pins() > 0, f"planted mistake {name} passed every pin"
