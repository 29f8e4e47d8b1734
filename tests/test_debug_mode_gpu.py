"""SAGESLA_DEBUG=1 on the GPU: a forward and a backward in a child process whose library synchronizes after every
stage return the same bits as the asynchronous run in this process. (The variable is read once per process, hence
the child; its injected-failure behaviour is covered on the host by test_abi_host_sanitized.)"""
import os
import subprocess
import sys

import pytest
import torch

import int8_block_sparse_amd as sg
import synth

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
import int8_block_sparse_amd as sg, synth
wl = synth.custom(1, 2, 1000, blk_q=128, topk_frac=0.25, name="debug-mode")
q, k, v, w = synth.make(wl, 3, device="cuda")
out = sg.forward(q, k, v, w, topk=wl.topk, blk_q=wl.blk_q)
dy = torch.randn(q.shape, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).cuda()
_, ex = sg.forward(q, k, v, w, topk=wl.topk, blk_q=wl.blk_q, export=True)
g = sg.backward(q, k, v, w, dy, ex["block_idx"][..., :wl.topk].contiguous(), topk=wl.topk)
torch.cuda.synchronize()
torch.save({"out": out.cpu(), "dq": g[0].cpu(), "dk": g[1].cpu(), "dv": g[2].cpu(), "dw": g[3].cpu()}, sys.argv[2])
print("child done", flush=True)
"""


def test_debug_mode_matches_async(tmp_path):
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    path = str(tmp_path / "debug.pt")
    env = dict(os.environ, SAGESLA_DEBUG="1")
    print("child: forward + backward with SAGESLA_DEBUG=1", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, path], env=env, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert "sagesla:" not in r.stderr
    got = torch.load(path, weights_only=True)
    sg.load()
    wl = synth.custom(1, 2, 1000, blk_q=128, topk_frac=0.25, name="debug-mode")
    q, k, v, w = synth.make(wl, 3, device="cuda")
    out = sg.forward(q, k, v, w, topk=wl.topk, blk_q=wl.blk_q)
    dy = torch.randn(q.shape, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).cuda()
    _, ex = sg.forward(q, k, v, w, topk=wl.topk, blk_q=wl.blk_q, export=True)
    g = sg.backward(q, k, v, w, dy, ex["block_idx"][..., :wl.topk].contiguous(), topk=wl.topk)
    torch.cuda.synchronize()
    assert torch.equal(got["out"], out.cpu())
    for i, name in enumerate(("dq", "dk", "dv", "dw")):
        assert torch.equal(got[name], g[i].cpu()), name
