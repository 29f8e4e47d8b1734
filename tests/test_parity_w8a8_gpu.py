"""GPU parity of the W8A8 linear layer (include/w8a8.h) against the fp64 oracle (oracle/w8a8.py).

Codes and scales must be bit-exact. The bf16 output must lie within the bound derived from the kernel's
arithmetic: fp32(s_x * s_w) and each fused multiply-add round with relative error 2^-24, so the fp32 sum
over n_kb k-blocks plus the bias is within (n_kb + 2) * 2^-24 * A of the exact value, A = sum |s_x s_w P| + |b|
(the oracle's abs_terms); rounding to bf16 then adds at most 2^-8 of the value. The test allows
2^-8 |y| + (n_kb + 3) * 2^-23 * A.
"""
import numpy as np
import pytest
import torch

import synth
from conftest import to_np
from oracle import w8a8 as ow

pytestmark = pytest.mark.gpu

SMALL = [
    synth.LinearWorkload("ragged-halfN", 300, 384, 640),  # 3 token tiles (last 44 rows), last output tile half
    synth.LinearWorkload("one-kblock", 129, 256, 128),    # K = 128: a single k-block; 1 valid row in tile 2
    synth.LinearWorkload("single-row", 1, 128, 384),
    synth.LinearWorkload("six-kblocks", 256, 512, 768),   # k-block count a multiple of the ring's unroll
    synth.LinearWorkload("seven-kblocks", 200, 640, 896),
]


def lib_w8a8():
    import int8_block_sparse_amd.w8a8 as w8
    return w8


def check_y(y_gpu, Y_ref, A, nkb):
    y = to_np(y_gpu)
    tol = 2.0 ** -8 * np.abs(Y_ref) + (nkb + 3) * 2.0 ** -23 * A
    err = np.abs(y - Y_ref)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} outputs outside the bound; worst excess {np.max(err - tol):.3e}"


def run_case(wl, seed, clip=1.0, bias=True):
    w8 = lib_w8a8()
    x, w, b = synth.make_linear(wl, seed, bias=bias)
    xg, wg = x.cuda(), w.cuda()
    bg = b.cuda() if b is not None else None
    wq_g, ws_g = w8.quantize(wg, 1.0)
    y = w8.linear(xg, wq_g, ws_g, bg, clip=clip)
    xq_g, xs_g = w8.quantize(xg, clip)
    torch.cuda.synchronize()
    Y, (xq, xs), (wq, ws) = ow.linear(to_np(x), to_np(w), None if b is None else to_np(b), clip)
    np.testing.assert_array_equal(wq_g.cpu().numpy(), wq)
    np.testing.assert_array_equal(ws_g.cpu().double().numpy(), ws)
    np.testing.assert_array_equal(xq_g.cpu().numpy(), xq)
    np.testing.assert_array_equal(xs_g.cpu().double().numpy(), xs)
    A = ow.abs_terms(xq, xs, wq, ws, None if b is None else to_np(b))
    check_y(y, Y, A, wl.K // 128)
    return y


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_linear_small(wl):
    run_case(wl, 0)


@pytest.mark.parametrize("clip", [0.5, 0.125])
def test_linear_clipped(clip):
    run_case(SMALL[0], 1, clip=clip)


def test_linear_no_bias_and_gemm_entry():
    w8 = lib_w8a8()
    wl = SMALL[4]
    y = run_case(wl, 2, bias=False)
    # the product from given codes equals the whole layer's output bit for bit
    x, w, _ = synth.make_linear(wl, 2, bias=False)
    xq, xs = w8.quantize(x.cuda())
    wq, ws = w8.quantize(w.cuda())
    y2 = w8.gemm(xq, xs, wq, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_zero_blocks_and_rows():
    w8 = lib_w8a8()
    wl = SMALL[0]
    x, w, b = synth.make_linear(wl, 3)
    x[:, 128:256] = 0  # a zero k-block column for every token tile
    x[290:] = 0        # zero rows in the ragged last tile
    w[128:256, 256:384] = 0
    xg, wg, bg = x.cuda(), w.cuda(), b.cuda()
    wq, ws = w8.quantize(wg)
    y = w8.linear(xg, wq, ws, bg)
    xq_g, xs_g = w8.quantize(xg)
    torch.cuda.synchronize()
    Y, (xq, xs), (wq_o, ws_o) = ow.linear(to_np(x), to_np(w), to_np(b))
    np.testing.assert_array_equal(xq_g.cpu().numpy(), xq)
    np.testing.assert_array_equal(xs_g.cpu().double().numpy(), xs)
    assert (xs[:, 1] == 0).all()
    check_y(y, Y, ow.abs_terms(xq, xs, wq_o, ws_o, to_np(b)), wl.K // 128)
    # rows with only zero inputs give exactly the bias
    np.testing.assert_array_equal(to_np(y[290:]), np.broadcast_to(to_np(b), (10, wl.N)))


@pytest.mark.parametrize("clip", [1.0, 0.5])
def test_power_of_two_scaling(clip):
    # exact for the arithmetic of the layer: X times 2^5 and W times 2^-2 leave every code as it is and scale each
    # block scale, each fp32 scale product, each fused multiply-add and the bf16 rounding by powers of two, so
    # (without a bias) the output must be 2^3 times the unscaled one bit for bit
    w8 = lib_w8a8()
    x, w, _ = synth.make_linear(SMALL[0], 9)
    xg, wg = x.cuda(), w.cuda()
    wq, ws = w8.quantize(wg)
    wq2, ws2 = w8.quantize((wg.float() * 0.25).to(torch.bfloat16))
    y1 = w8.linear(xg, wq, ws, None, clip=clip)
    y2 = w8.linear((xg.float() * 32).to(torch.bfloat16), wq2, ws2, None, clip=clip)
    torch.cuda.synchronize()
    assert torch.equal(wq2, wq) and torch.equal(ws2, ws * 0.25)
    assert torch.equal(y2.float(), y1.float() * 8)


def test_deterministic():
    w8 = lib_w8a8()
    x, w, b = synth.make_linear(SMALL[4], 4)
    xg, wg, bg = x.cuda(), w.cuda(), b.cuda()
    wq, ws = w8.quantize(wg)
    y1 = w8.linear(xg, wq, ws, bg, clip=0.9)
    y2 = w8.linear(xg, wq, ws, bg, clip=0.9)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def sampled_full(name, rows_blocks, n_cols, seed=0, clip=1.0):
    """Full-size layer on the GPU; the oracle checks whole token blocks (codes, scales, outputs) on sampled output
    columns."""
    w8 = lib_w8a8()
    wl = synth.LINEAR_WORKLOADS[name]
    x, w, b = synth.make_linear(wl, seed, device="cuda")
    print(f"[w8a8 full] {name} M={wl.M} N={wl.N} K={wl.K} clip={clip}", flush=True)
    wq_g, ws_g = w8.quantize(w)
    y = w8.linear(x, wq_g, ws_g, b, clip=clip)
    xq_g, xs_g = w8.quantize(x, clip)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([rng.choice(wl.N, n_cols, replace=False), [0, wl.N - 1]]))
    W = to_np(w)
    wq_o, ws_o = ow.quantize_blocks(W)
    np.testing.assert_array_equal(wq_g.cpu().numpy(), wq_o)
    np.testing.assert_array_equal(ws_g.cpu().double().numpy(), ws_o)
    nmb = ow.n_blocks(wl.M)
    for mb in rows_blocks:
        mb = mb % nmb
        r0, r1 = mb * 128, min(wl.M, mb * 128 + 128)
        xq, xs = ow.quantize_blocks(to_np(x[r0:r1]), clip)
        np.testing.assert_array_equal(xq_g[r0:r1].cpu().numpy(), xq)
        np.testing.assert_array_equal(xs_g[mb].cpu().double().numpy(), xs[0])
        wsel = wq_o[cols]
        wss = ws_o[cols // 128]  # the scale rows of the sampled output columns
        bb = to_np(b)[cols]
        Y = np.zeros((r1 - r0, len(cols)))
        A = np.zeros_like(Y)
        for kb in range(wl.K // 128):
            sl = slice(kb * 128, kb * 128 + 128)
            P = xq[:, sl].astype(np.int64) @ wsel[:, sl].astype(np.int64).T
            c = xs[0, kb] * wss[:, kb]
            Y += c[None, :] * P
            A += np.abs(c[None, :] * P)
        Y += bb[None, :]
        A += np.abs(bb)[None, :]
        check_y(y[r0:r1][:, torch.from_numpy(cols).cuda()], Y, A, wl.K // 128)


def test_full_size_720p_proj():
    sampled_full("wan14b-720p-proj", [0, 517, -1], 192)


def test_full_size_720p_ffn_down_clipped():
    sampled_full("wan14b-720p-ffn-down", [3, -1], 128, seed=1, clip=0.8)


@pytest.mark.timeout(600)
def test_full_size_ffn_down_max_rows():
    # the largest activation matrix the limits allow for 13824 inputs (155344 tokens: 2^31 - 8192 elements, the
    # last token block ragged; one more token is refused, which the host-side checks of the C ABI test)
    wl = synth.LINEAR_WORKLOADS["wan14b-ffn-down-max-rows"]
    assert wl.M * wl.K < 2 ** 31 <= (wl.M + 1) * wl.K
    sampled_full("wan14b-ffn-down-max-rows", [0, 600, -2, -1], 96, seed=2)
