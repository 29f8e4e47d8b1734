"""The entry points under HIP graph capture: sagesla_forward and sagesla_backward, captured once with caller-owned
outputs and workspace, are replayed three times with eager work and synchronizations in between, and every replay
must reproduce the eager result bit for bit (the library allocates nothing, clears with kernels rather than memset
nodes, and is deterministic). The attention entry points are also captured with the RMSNorm of Q and K in front."""
import pytest
import torch

import int8_block_sparse_amd as sg
import synth

pytestmark = pytest.mark.gpu


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one warm-up call off the capture, as torch recommends
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    return g, res


def eager_noise():
    x = torch.randn(1 << 20, device="cuda")
    return float((x * x).sum())  # eager kernels and a synchronization between the replays


def norm_weights(H, D, use):
    """(gamma_q, gamma_k, eps) for the RMSNorm of Q and K, or None."""
    if not use:
        return None
    gen = torch.Generator().manual_seed(5)
    gq, gk = ((1 + 0.2 * torch.randn(H * D, generator=gen)).to(torch.bfloat16).cuda() for _ in range(2))
    return gq, gk, 1e-6


@pytest.mark.parametrize("use_norm", [False, True])
def test_forward_replays(use_norm):
    wl = synth.custom(1, 2, 1000, blk_q=128, topk_frac=0.2)
    q, k, v, w = (t.cuda() for t in synth.make(wl, 0))
    norm = norm_weights(wl.H, wl.D, use_norm)
    cfg = sg.Config(wl.B, wl.H, wl.N, wl.D, wl.blk_q, wl.blk_k, wl.topk, wl.linear, qk_norm=use_norm)
    ws = torch.empty(sg.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    ref = sg.forward(q, k, v, w, topk=wl.topk, workspace=ws, norm=norm).clone()
    out = torch.empty_like(q)
    g, _ = capture(lambda: sg.forward(q, k, v, w, topk=wl.topk, out=out, workspace=ws, norm=norm))
    for _ in range(3):
        out.fill_(0)
        eager_noise()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


@pytest.mark.parametrize("use_norm", [False, True])
def test_backward_replays(use_norm):
    wl = synth.custom(1, 2, 1000, blk_q=128, topk_frac=0.2)
    q, k, v, w = (t.cuda() for t in synth.make(wl, 1))
    norm = norm_weights(wl.H, wl.D, use_norm)
    dy = torch.randn(q.shape, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).cuda()
    _, ex = sg.forward(q, k, v, w, topk=wl.topk, export=True, norm=norm)
    sel = ex["block_idx"][..., :wl.topk].contiguous()
    cfg = sg.Config(wl.B, wl.H, wl.N, wl.D, wl.blk_q, wl.blk_k, wl.topk, wl.linear, qk_norm=use_norm)
    import ctypes
    nargs = {} if norm is None else {"q_norm_w": norm[0].data_ptr(), "k_norm_w": norm[1].data_ptr(),
                                     "norm_eps": norm[2]}
    need = sg.load().sagesla_backward_workspace_bytes(ctypes.byref(cfg.params(w_proj=w.data_ptr(), **nargs)))
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref = [t.clone() for t in sg.backward(q, k, v, w, dy, sel, topk=wl.topk, workspace=ws, norm=norm)]
    g, got = capture(lambda: sg.backward(q, k, v, w, dy, sel, topk=wl.topk, workspace=ws, norm=norm))
    for _ in range(3):
        for t in got:
            t.fill_(0)
        eager_noise()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)


def test_w8a8_linear_replays():
    import int8_block_sparse_amd.w8a8 as w8
    wl = synth.LinearWorkload("graph", 300, 384, 640)
    x, w, b = (t.cuda() for t in synth.make_linear(wl, 3))
    wq, wsc = w8.quantize(w)
    ws = torch.empty(w8.workspace_bytes(wl.M, wl.K), dtype=torch.uint8, device="cuda")
    ref = w8.linear(x, wq, wsc, b, clip=0.9, workspace=ws).clone()
    y = torch.empty_like(ref)
    g, _ = capture(lambda: w8.linear(x, wq, wsc, b, clip=0.9, out=y, workspace=ws))
    for _ in range(3):
        y.fill_(0)
        eager_noise()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
