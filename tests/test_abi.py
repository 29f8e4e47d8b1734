"""The C-ABI library: it loads, exports every entry point its header declares, its parameter block has the
layout a C compiler gives it, and host-side validation returns the documented status codes without launching
anything. CPU only (no kernel is called)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import int8_block_sparse_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sagesla.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sg.LIB_PATH):
        pytest.fail("libsagesla.so is not built (run __graft_entry__.build())")
    return sg.load()


def declared_functions():
    """Every function declared by the headers under include/ (prototypes: a return type, a name, a parameter
    list ending in ';')."""
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b((?:sagesla|w8a8)_[a-z0-9_]+)\s*\([^;{]*\)\s*;", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"sagesla_quantize", "sagesla_select", "sagesla_forward", "sagesla_workspace_bytes", "w8a8_quantize",
            "w8a8_gemm", "w8a8_linear", "w8a8_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_param_block_layout_matches_c(tmp_path):
    fields = [f for f, _ in sg.Params._fields_]
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "sagesla.h"\nint main(void){\n'
        '  printf("%zu", sizeof(sagesla_params));\n'
        + "".join(f'  printf(" %zu", offsetof(sagesla_params, {f}));\n' for f in fields)
        + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(sg.Params)] + [getattr(sg.Params, f).offset for f in fields]
    assert got == want


def test_status_strings(lib):
    for code in range(7):
        assert lib.sagesla_status_str(code)
    assert lib.sagesla_last_hip_error() == 0


# Validation must reject these before touching the device. The fake pointers below are never dereferenced on
# the host; the tests are skipped where a GPU is visible so a validation bug can never launch with them.
try:
    import torch
    _gpu = torch.cuda.is_available()
except Exception:  # noqa: BLE001
    _gpu = False
cpu_only = pytest.mark.skipif(_gpu, reason="host-validation tests use fake device pointers; CPU only")

FAKE = 1 << 40  # 256-byte aligned, never dereferenced


def good(**kw):
    cfg = sg.Config(B=1, H=2, N=1000, blk_q=128, blk_k=64, topk=2, linear=True)
    p = cfg.params(w_proj=FAKE, workspace=FAKE, workspace_bytes=1 << 40)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def fwd(lib, p, q=FAKE, k=FAKE, v=FAKE, out=FAKE):
    return lib.sagesla_forward(q, k, v, out, ctypes.byref(p), None)


@cpu_only
@pytest.mark.parametrize("field,value,status", [
    ("D", 64, 3), ("blk_k", 128, 3), ("blk_q", 32, 3), ("flags", 0x20, 3), ("N", (1 << 24) + 1, 3),
    ("B", 0, 2), ("H", 0, 2), ("N", 0, 2), ("topk", -1, 2), ("topk", 17, 2), ("B", 300, 2),
    ("sm_scale", float("nan"), 2), ("sm_scale", -1.0, 2),
    ("w_proj", None, 1), ("workspace", None, 4), ("workspace_bytes", 100, 4),
    ("workspace", FAKE + 16, 5), ("q_i8", FAKE + 8, 5), ("o_lin", FAKE + 4, 5), ("w_proj", FAKE + 2, 5),
])
def test_forward_validation(lib, field, value, status):
    p = good(**{field: value})
    if field == "B":
        p.H = 300 if value == 300 else p.H
    assert fwd(lib, p) == status


@cpu_only
def test_norm_validation(lib):
    p = good(flags=sg.LINEAR | sg.QK_RMSNORM, q_norm_w=FAKE, k_norm_w=FAKE, norm_eps=1e-6)
    assert lib.sagesla_validate(ctypes.byref(p)) == 0
    assert lib.sagesla_validate(ctypes.byref(good(flags=sg.LINEAR | sg.QK_RMSNORM, k_norm_w=FAKE))) == 1
    assert lib.sagesla_validate(ctypes.byref(good(flags=sg.LINEAR | sg.QK_RMSNORM, q_norm_w=FAKE,
                                                  k_norm_w=FAKE, norm_eps=-1.0))) == 2
    assert lib.sagesla_validate(ctypes.byref(good(flags=sg.LINEAR | sg.QK_RMSNORM, q_norm_w=FAKE + 2,
                                                  k_norm_w=FAKE))) == 5
    assert lib.sagesla_validate(ctypes.byref(good(flags=sg.LINEAR | sg.QK_RMSNORM, q_norm_w=FAKE, k_norm_w=FAKE,
                                                  q_hat=FAKE + 8))) == 5
    # the norm's two [B][H][N][D] bf16 copies live in the workspace
    cfg = sg.Config(B=1, H=2, N=1000, topk=2, linear=True)
    plain = lib.sagesla_workspace_bytes(ctypes.byref(cfg.params()))
    cfg.qk_norm = True
    assert lib.sagesla_workspace_bytes(ctypes.byref(cfg.params())) >= plain + 2 * 2 * 1000 * 128 * 2


@cpu_only
def test_tensor_pointer_validation(lib):
    assert fwd(lib, good(), q=None) == 1
    assert fwd(lib, good(), out=None) == 1
    assert fwd(lib, good(), v=FAKE + 2) == 5
    p = good(flags=sg.LINEAR | sg.USE_GIVEN_MASK)
    assert fwd(lib, p) == 1  # given mask without block_idx
    p = good()
    assert lib.sagesla_quantize(None, FAKE, ctypes.byref(p), None) == 1
    p = good(D=96)
    assert lib.sagesla_select(ctypes.byref(p), None) == 3
    assert lib.sagesla_last_hip_error() == 0


@cpu_only
def test_forward_noalloc_validation(lib):
    # the same checks as sagesla_forward, then the plan against the library's scratch, all before any device call
    nf = lambda p, q=FAKE, out=FAKE: lib.sagesla_forward_noalloc(q, FAKE, FAKE, out, ctypes.byref(p), None)
    assert nf(good(D=64)) == 3 and nf(good(topk=-1)) == 2 and nf(good(w_proj=None)) == 1
    assert nf(good(), q=None) == 1 and nf(good(), out=FAKE + 2) == 5
    assert nf(good(flags=sg.LINEAR | sg.USE_GIVEN_MASK)) == 1
    big = sg.Config(B=1, H=12, N=32760, topk=51, linear=True).params(w_proj=FAKE)
    assert lib.sagesla_workspace_bytes(ctypes.byref(big)) > sg.NOALLOC_SCRATCH_BYTES
    assert nf(big) == 4  # more than the scratch holds
    assert lib.sagesla_last_hip_error() == 0


def bwd(lib, p, dq=FAKE, dk=FAKE, dv=FAKE, dw=FAKE, q=FAKE):
    return lib.sagesla_backward(q, FAKE, FAKE, FAKE, dq, dk, dv, dw, ctypes.byref(p), None)


@cpu_only
def test_backward_validation(lib):
    ok = dict(block_idx=FAKE)
    need = lib.sagesla_backward_workspace_bytes(ctypes.byref(good(**ok)))
    assert need > lib.sagesla_workspace_bytes(ctypes.byref(good(**ok)))  # fp32 states, O_l and the gradients' buffers
    assert bwd(lib, good()) == 1                       # topk > 0 without a selection
    assert bwd(lib, good(**ok), dq=None) == 1
    assert bwd(lib, good(**ok), q=None) == 1
    assert bwd(lib, good(**ok), dw=None) == 1          # the linear branch needs dW_p
    assert bwd(lib, good(**ok), dk=FAKE + 4) == 5
    assert bwd(lib, good(workspace_bytes=need - 1, **ok)) == 4
    assert bwd(lib, good(workspace=FAKE + 16, **ok)) == 5
    norm = good(flags=sg.LINEAR | sg.QK_RMSNORM, q_norm_w=FAKE, k_norm_w=FAKE, norm_eps=1e-6, **ok)
    assert bwd(lib, norm) == 1                         # the norm needs its weight-gradient outputs
    norm.dq_norm_w, norm.dk_norm_w = FAKE, FAKE + 4
    assert bwd(lib, norm) == 5
    norm.dk_norm_w = FAKE
    assert lib.sagesla_backward_workspace_bytes(ctypes.byref(norm)) > need  # normalized copies, norm partials
    assert bwd(lib, good(D=64, **ok)) == 3
    assert lib.sagesla_last_hip_error() == 0


def test_workspace_bytes(lib):
    cfg = sg.Config(B=2, H=40, N=75600, blk_q=128, blk_k=64, topk=118, linear=True)
    n = lib.sagesla_workspace_bytes(ctypes.byref(cfg.params()))
    # int8 codes of Q and K alone are 2*B*H*N*D bytes; the linear branch adds states, remainders and O_lin
    assert n > 2 * 2 * 40 * 75600 * 128
    assert n < 32 << 30
    cfg_dense = sg.Config(B=1, H=12, N=32760, blk_q=128, blk_k=64, topk=512, linear=False)
    assert 0 < lib.sagesla_workspace_bytes(ctypes.byref(cfg_dense.params())) < n
    bad = sg.Config(B=1, H=1, N=100, D=64)
    assert lib.sagesla_workspace_bytes(ctypes.byref(bad.params())) == 0
    # key-block count: up to 20480 with or without the linear branch
    big = sg.Config(B=1, H=1, N=64 * 12000, topk=10, linear=True)
    assert lib.sagesla_validate(ctypes.byref(big.params(w_proj=FAKE))) == 0
    big.linear = False
    assert lib.sagesla_validate(ctypes.byref(big.params())) == 0
    huge = sg.Config(B=1, H=1, N=64 * 20481, topk=10, linear=True)
    assert lib.sagesla_validate(ctypes.byref(huge.params(w_proj=FAKE))) == 3


def test_topk_blocks_matches_flag_reading():
    assert [sg.topk_blocks(f, n) for f, n in [(0.25, 16), (1.0, 512), (0.1, 512), (0.1, 1182), (0.05, 4208)]] == \
        [4, 512, 51, 118, 210]


# ---------------------------------------------------------------------------------------------------------
# W8A8 linear layer (include/w8a8.h): host-side validation only
# ---------------------------------------------------------------------------------------------------------
@cpu_only
@pytest.mark.parametrize("rows,cols,clip,status", [
    (0, 128, 1.0, 2), (4, 0, 1.0, 2), (4, 128, 0.0, 2), (4, 128, 1.5, 2), (4, 128, float("nan"), 2),
    (4, 100, 1.0, 3), ((1 << 24) + 1, 128, 1.0, 3), (1 << 17, 1 << 14, 1.0, 3),
])
def test_w8a8_quantize_validation(lib, rows, cols, clip, status):
    assert lib.w8a8_quantize(FAKE, rows, cols, clip, FAKE, FAKE, None) == status


@cpu_only
def test_w8a8_pointer_validation(lib):
    assert lib.w8a8_quantize(None, 4, 128, 1.0, FAKE, FAKE, None) == 1
    assert lib.w8a8_quantize(FAKE + 2, 4, 128, 1.0, FAKE, FAKE, None) == 5
    g = lambda **kw: lib.w8a8_gemm(kw.get("x", FAKE), FAKE, FAKE, FAKE, kw.get("b", None), kw.get("y", FAKE),
                                   kw.get("M", 300), kw.get("N", 256), kw.get("K", 384), None)
    assert g(x=None) == 1 and g(y=None) == 1 and g(b=FAKE + 8) == 5 and g(y=FAKE + 4) == 5
    assert g(N=200) == 3 and g(K=200) == 3 and g(K=32768 + 128) == 3 and g(M=0) == 2
    lin = lambda **kw: lib.w8a8_linear(FAKE, FAKE, FAKE, None, FAKE, 300, 256, 384, kw.get("clip", 1.0),
                                       kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    assert lin(clip=0.0) == 2 and lin(ws=None) == 4 and lin(wsb=1000) == 4 and lin(ws=FAKE + 16) == 5
    assert lib.sagesla_last_hip_error() == 0


def test_w8a8_workspace_bytes(lib):
    assert lib.w8a8_workspace_bytes(300, 384) == 115200 + 256  # codes (aligned) + 3 x 3 scales (aligned)
    assert lib.w8a8_workspace_bytes(151200, 5120) >= 151200 * 5120
    assert lib.w8a8_workspace_bytes(0, 128) == 0 and lib.w8a8_workspace_bytes(10, 100) == 0
