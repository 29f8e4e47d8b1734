"""sagesla_forward_noalloc (the forward for callers that cannot allocate: its workspace is the library's own
device scratch) against sagesla_forward through the C ABI: identical outputs and intermediates on two calls in a
row, the second on a smaller layer, so the second call runs on scratch the first one left behind."""
import pytest
import torch

import int8_block_sparse_amd as sg
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    sg.load()


def say(*a):
    print(*a, flush=True)


CASES = [
    # (workload, seed, group32): the largest first (about 42 MiB of the 64 MiB scratch), then a small ragged one
    (synth.custom(1, 4, 8192, grid=(8, 32, 32), structured=True, blk_q=128, topk_frac=0.1, name="noalloc-8k"), 0,
     False),
    (synth.custom(2, 1, 1000, blk_q=64, topk_frac=0.2, name="noalloc-ragged"), 1, True),
]


def test_noalloc_matches_forward_on_two_calls():
    for wl, seed, g32 in CASES:
        cfg = sg.Config(wl.B, wl.H, wl.N, wl.D, wl.blk_q, wl.blk_k, wl.topk, wl.linear, group32=g32)
        need = sg.workspace_bytes(cfg)
        say(f"case {wl.name} B{wl.B} H{wl.H} N{wl.N} bq{wl.blk_q} topk {wl.topk} group32 {g32}: "
            f"plan {need / 2**20:.1f} MiB")
        assert need <= sg.NOALLOC_SCRATCH_BYTES
        q, k, v, w = synth.make(wl, seed, device="cuda")
        ref, exr = sg.forward(q, k, v, w, topk=wl.topk, blk_q=wl.blk_q, export=True, group32=g32)
        got, exg = sg.forward_noalloc(q, k, v, w, topk=wl.topk, blk_q=wl.blk_q, export=True, group32=g32)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{wl.name}: outputs differ"
        for name in exr:
            assert torch.equal(exg[name], exr[name]), f"{wl.name}: {name} differs"
        say(f"  identical: out and {len(exr)} intermediates")


def test_noalloc_refuses_a_layer_beyond_the_scratch():
    wl = synth.custom(1, 12, 32760, blk_q=128, topk_frac=0.1, name="too-big")
    q = torch.zeros(1, 12, 32760, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(128, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sg.SageSLAError, match="E_WORKSPACE"):
        sg.forward_noalloc(q, q, q, w, topk=wl.topk)
