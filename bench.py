"""Benchmark of the SageSLA attention forward on one MI355X.

A step is one whole forward (quantize, select, linear branch, sparse attention) of the Wan2.1-14B-720P layer
shape as a conditional/unconditional pair: B=2, H=40, N=75600 (21×45×80 latent tokens), D=128, blocks 128×64,
top-k 10% (118 of 1182 key blocks), on seeded synthetic inputs already resident in HBM.

Prints one JSON line: the metric ms/layer with dense-equivalent TOPS as `value`, the sparse-attention kernel's
roofline (its duration measured with HIP events recorded by the library around it on the launch stream), and
the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--calib-copy-mib M] [--workload W]

The other seeded forward shapes print the same line with --workload <name>: wan1.3b-480p-dense (dense INT8
attention, linear branch off), wan1.3b-480p-sla (the 1.3B 480P layer at top-k 10%), 1080p-long-sla (N=269280,
top-k 5%) and tiny.

The second workload, the W8A8 block-quantized linear layer ("Turbo Diffusion", lanhy.cn, §三(四) item 1), is
measured with --workload w8a8-<shape> (shapes: the synth module's LINEAR_WORKLOADS, e.g. w8a8-wan14b-720p-proj):
a step is one whole layer (activation quantization, then the block-scaled INT8 product with the pre-quantized
weights) and the line carries the product kernel's roofline.

--workload sla-backward times sagesla_backward (SLA is trainable, §三(二)) on the same 720P pair for the
forward's own selection; a step is one whole backward (every kernel of it).

The headline line also reports a cold variant: the median forward time when a 512 MiB device fill (twice the
Infinity Cache) precedes each forward.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SageSLA fwd ms/layer + dense-equiv TOPS (% INT8 MFMA peak), N=75600 H=40 D=128"
WORKLOAD = 3  # the 14B-720P pair: the configuration the metric is quoted on
HEADLINE = "wan14b-720p-sla-pair"
PEAK_INT8_TOPS = 5000.0  # MI355X dense INT8 MFMA
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
# Layouts of the forward's linear branch as the kernels store them: the fp16 state table (H_J^T and Z_J per key
# block, with the block's exponent) and the remaining state of each query block (the fp16 plane of H_m^T, then Z_m
# and the plane rows' factors in fp32)
STATE_BYTES_PER_BLOCK = (128 * 128 + 128) * 2 + 4
REMAINING_BYTES_PER_QBLOCK = 128 * 128 * 2 + 2 * 128 * 4
# products of bq x D x D per query block in the attention kernel's linear epilogue: phi(Q) H_m (one fp16 product),
# then (.) W_p on the bf16 hi and lo halves of the first result
EPILOGUE_PRODUCTS_EXECUTED = 3
# whole heads the CPU baseline runs per workload (about 10-30 s of oracle time each); on the longest layer one
# head's attention outputs are formed for a sample of its query blocks only
CPU_HEADS = {"tiny": 2, "wan1.3b-480p-dense": 4, "wan1.3b-480p-sla": 6, "wan14b-720p-sla-pair": 2,
             "1080p-long-sla": 1}
CPU_BLOCKS = {"1080p-long-sla": 128}
CSRC = os.path.join(ROOT, "int8_block_sparse_amd", "csrc")
COUNTERS = os.path.join(ROOT, "profiles", "forward_hbm_wan14b-720p-sla-pair.txt")
K3_SOURCE = os.path.join(CSRC, "k_attn.hip")
# the kernels whose HBM traffic the headline line reports from the committed counter summary, with their sources
HBM_KERNELS = {"k3_attn<4, false>": "k_attn.hip", "k1_quant<128, false>": "k_quant.hip", "k4_gemm16": "k_linear.hip"}
W8A8_COUNTERS = os.path.join(ROOT, "profiles", "k5_gemm_wan14b-720p-proj_counters.txt")
W8A8_SOURCE = os.path.join(ROOT, "int8_block_sparse_amd", "csrc", "k_w8a8.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _summary_kv(path):
    kv = {}
    for line in open(path):
        if ": " in line and not line.startswith("#"):
            k, v = line.rsplit(": ", 1)  # keys may hold ':' themselves ("sha256[:16]")
            kv[k.strip()] = v.strip()
    return kv


def read_counters(path=COUNTERS, source=K3_SOURCE, kernel=None):
    """HBM bytes per launch of a kernel (default: the summary's dominant kernel) from a committed rocprofv3
    counter summary, or None when absent or taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    kv = _summary_kv(path)
    if kv.get(f"{os.path.basename(source)} sha256[:16]") != source_sha(source):
        return None
    key = (f"{kernel} hbm bytes per launch (fetch+write, copy-calibrated)" if kernel
           else "hbm bytes per launch (fetch+write, copy-calibrated)")
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def read_kernel_hbm(path=COUNTERS):
    """Per-kernel HBM bytes and kernel-trace time per launch of the forward's bandwidth-bound kernels from the
    committed counter summary; a kernel whose source changed since is left out."""
    if not os.path.exists(path):
        return {}
    kv = _summary_kv(path)
    out = {}
    for kern, src in HBM_KERNELS.items():
        if kv.get(f"{src} sha256[:16]") != source_sha(os.path.join(CSRC, src)):
            continue
        try:
            byt = float(kv[f"{kern} hbm bytes per launch (fetch+write, copy-calibrated)"])
            ms = float(kv[f"{kern} average launch (kernel trace) ms"])
        except (KeyError, ValueError):
            continue
        out[kern] = {"hbm_bytes": byt, "ms": ms, "achieved_GBps": round(byt / ms / 1e6, 1),
                     "frac": round(byt / ms / 1e6 / PEAK_HBM_GBPS, 4)}
    return out


MFMA_COUNTERS = os.path.join(ROOT, "profiles", "k3_attn_wan14b-720p-sla-pair_mfma_counters.txt")


def read_mfma_util(path=MFMA_COUNTERS, source=K3_SOURCE):
    """MFMA busy fraction of the attention kernel (busy cycles over active cycles, at the clock the box holds)
    from its committed rocprofv3 counter summary, or None when absent or taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ": " in line and not line.startswith("#"):
            k, v = line.rsplit(": ", 1)
            kv[k.strip()] = v.strip()
    if kv.get(f"{os.path.basename(source)} sha256[:16]") != source_sha(source):
        return None
    for k, v in kv.items():
        if k.startswith("k3_attn<4, false> MfmaUtil"):
            try:
                return float(v)
            except ValueError:
                return None
    return None


def host_info():
    """The host CPU model and the BLAS numpy runs the oracle's products on (library, version, threads)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            i = infos[0]
            blas = f"{i.get('internal_api', '?')} {i.get('version', '?')} ({i.get('threading_layer', '?')})"
            threads = max(j.get("num_threads", 1) for j in infos)
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "blas": blas, "blas_threads": int(threads),
            "affinity_cores": len(os.sched_getaffinity(0))}


def selection_check(r, scores, idx, D):
    """The GPU's selection of one head against the oracle's: rows whose block list differs (each must be a near-tie
    row, gap below NEAR_TIE), near-tie rows, and the largest score difference, also as a fraction of the fp64
    rounding bound of the two sums (2^-44 |q_pool| . |k_pool|, both in the oracle's 1/sqrt(D) units)."""
    import numpy as np
    from oracle import sagesla as orc
    got = idx[:, :r["idx"].shape[1]]
    differ = np.any(got != r["idx"], axis=1)
    near = r["gap"] < orc.NEAR_TIE
    sg_ = scores / math.sqrt(D)
    bound = 2.0 ** -44 * (np.abs(r["q_pool"]) @ np.abs(r["k_pool"]).T) / math.sqrt(D) + 1e-300
    diff = np.abs(sg_ - r["scores"])
    return {"rows": int(len(differ)), "rows_differ": int(differ.sum()), "rows_differ_not_near_tie":
            int((differ & ~near).sum()), "near_tie_rows": int(near.sum()), "max_abs_score_diff": float(diff.max()),
            "max_diff_over_bound": float((diff / bound).max())}


def cpu_baseline(q, k, v, w, wl, heads, budget_s=30.0, blocks=None, gpu_sel=None):
    """The fp64 oracle (unchanged, untuned) on whole heads of the same workload; dense-equivalent TOPS.

    blocks: if given, each head's attention outputs are formed for that many evenly spaced query blocks only (its
    quantization, selection and linear-branch states still in full), and the dense-equivalent work is counted for
    those blocks' rows. gpu_sel: {(b, h): (scores, block lists)} exported by the GPU for those heads; the oracle's
    selection of each head is then compared with it (selection_check), outside the timed oracle work."""
    from oracle import sagesla as orc
    hi = host_info()
    checks = []
    cores = hi["blas_threads"]
    W = w.float().cpu().double().numpy()
    done, t0 = 0, time.perf_counter()
    sel = None if blocks is None else sorted(set(int(x) for x in
                                                 [round(i * (wl.n_qb - 1) / max(1, blocks - 1)) for i in range(blocks)]))
    for (b, h) in heads:
        Q = q[b, h].float().cpu().double().numpy()
        K = k[b, h].float().cpu().double().numpy()
        V = v[b, h].float().cpu().double().numpy()
        t1 = time.perf_counter()
        r = orc.forward_head(Q, K, V, W, wl.blk_q, wl.blk_k, wl.topk, linear=wl.linear, blocks=sel)
        t_or = time.perf_counter() - t1
        if gpu_sel is not None and (b, h) in gpu_sel:
            checks.append(selection_check(r, *gpu_sel[(b, h)], wl.D))
        t0 += time.perf_counter() - t1 - t_or  # the check is not oracle time
        done += 1
        log(f"cpu baseline: head {done}/{len(heads)} at {time.perf_counter() - t0:.1f} s")
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    rows = wl.N if sel is None else sum(min(wl.N, (I + 1) * wl.blk_q) - I * wl.blk_q for I in sel)
    ops = done * 4.0 * rows * wl.N * wl.D
    what = (f"each a full forward over all {wl.n_qb} query blocks" if sel is None else
            f"each with its quantization, selection and linear-branch states in full and the outputs of {len(sel)} of "
            f"its {wl.n_qb} query blocks (evenly spaced), counted as {rows} of {wl.N} rows")
    out = {"value": ops / dt / 1e12, "unit": "TOPS (dense-equivalent)", "cores": int(cores), "kind": "oracle",
           "sample": f"{done} of {wl.B * wl.H} (b,h) heads, {what}", "seconds": round(dt, 2), **hi}
    if checks:
        out["selection_check"] = {"heads": len(checks), **{key: (max if key.startswith("max") else sum)(
            c[key] for c in checks) for key in checks[0]}}
    return out


def cpu_baseline_w8a8(x, w, bias, wl, rows, budget_s=30.0):
    """The fp64 W8A8 oracle (unchanged, untuned) on whole 128-token blocks of the same layer; TOPS."""
    import numpy as np
    from oracle import w8a8 as ow
    hi = host_info()
    cores = hi["blas_threads"]
    W = w.float().cpu().double().numpy()
    b = bias.float().cpu().double().numpy()
    wq, ws = ow.quantize_blocks(W)  # one-time weight quantization: not timed
    done, t0 = 0, time.perf_counter()
    for r0 in range(0, rows, 128):
        X = x[r0:r0 + 128].float().cpu().double().numpy()
        xq, xs = ow.quantize_blocks(X)
        ow.block_gemm(xq, xs, wq, ws, b)
        done += X.shape[0]
        log(f"cpu baseline: {done}/{rows} tokens at {time.perf_counter() - t0:.1f} s")
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    del np
    return {"value": done * 2.0 * wl.N * wl.K / dt / 1e12, "unit": "TOPS (2*M*N*K per layer)", "cores": int(cores),
            "kind": "oracle", "sample": f"{done} of {wl.M} tokens (whole 128-token blocks), all {wl.N} outputs",
            "seconds": round(dt, 2), **hi}


def cpu_baseline_backward(q, k, v, w, dy, sel, wl, budget_s=20.0):
    """The fp64 backward oracle (unchanged, untuned) on whole query blocks of head (0, 0): the dQ rows of each
    block through that block's forward (its selected blocks and its linear branch); TFLOP/s counted like the
    GPU line (the five sparse-branch products of the block's selected pairs)."""
    from oracle import sla_backward as ob
    hi = host_info()
    cores = len(os.sched_getaffinity(0))
    try:
        import torch
        cores = torch.get_num_threads()
    except Exception:  # noqa: BLE001
        pass
    hi["torch_threads"] = int(cores)
    f = lambda t: t.float().cpu().double().numpy()
    Q, K, V, W, dY = f(q[0, 0]), f(k[0, 0]), f(v[0, 0]), f(w), f(dy[0, 0])
    idx = sel[0, 0].cpu().numpy()
    done, t0 = 0, time.perf_counter()
    while done < wl.n_qb:
        ob.dq_blocks(Q, K, V, W, idx, dY, wl.blk_q, wl.blk_k, [done], linear=wl.linear)
        done += 1
        log(f"cpu baseline: query block {done} at {time.perf_counter() - t0:.1f} s")
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = done * wl.topk * 5 * 2.0 * wl.blk_q * wl.blk_k * wl.D
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s (5 products of 2*bq*bk*D per selected block pair)",
            "cores": int(cores), "kind": "oracle",
            "sample": f"dQ rows of {done} whole query blocks of head (0, 0) (each through its own forward, the linear "
                      f"branch included, which dominates the oracle's time)",
            "seconds": round(dt, 2), **hi}


def main_w8a8(args, name):
    import torch
    import int8_block_sparse_amd as sg
    import int8_block_sparse_amd.w8a8 as w8
    import synth

    if name not in synth.LINEAR_WORKLOADS:
        sys.exit(f"unknown W8A8 shape {name}; one of {sorted(synth.LINEAR_WORKLOADS)}")
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    sg.load()
    dev = torch.device("cuda:0")
    wl = synth.LINEAR_WORKLOADS[name]
    log(f"generating {wl.name} inputs on the GPU")
    x, w, bias = synth.make_linear(wl, 0, device=dev)
    wq, wsc = w8.quantize(w)  # weights are quantized once, outside the timed steps
    y = torch.empty(wl.M, wl.N, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(w8.workspace_bytes(wl.M, wl.K), dtype=torch.uint8, device=dev)
    x8 = ws[:wl.M * wl.K].view(torch.int8).view(wl.M, wl.K)  # the layer's activation codes live in the workspace
    off = (wl.M * wl.K + 255) // 256 * 256
    xs = ws[off:off + 4 * w8.n_blocks(wl.M) * (wl.K // 128)].view(torch.float32).view(w8.n_blocks(wl.M), wl.K // 128)
    step = lambda: w8.linear(x, wq, wsc, bias, clip=1.0, out=y, workspace=ws)
    for _ in range(args.warmup):
        step()
    # per-kernel times: the two launches of one step, bracketed by events on the launch stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        w8.quantize(x, 1.0, x8, xs)
        ev[i][1].record()
        w8.gemm(x8, xs, wq, wsc, bias, out=y)
        ev[i][2].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    t_q = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    t_g = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    log(f"{ms:.3f} ms/layer; quantize {t_q:.3f} ms, gemm {t_g:.3f} ms")
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        a2 = torch.empty_like(a)
        a2.copy_(a)
        torch.cuda.synchronize()
    ops = wl.ops
    gemm_tops = ops / (t_g * 1e-3) / 1e12
    result = {
        "metric": "W8A8 block-quantized linear layer TOPS (2*M*N*K per layer, INT8 MFMA)",
        "value": round(ops / (ms * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K, "block": 128, "clip": 1.0, "bias": True,
                   "parallelism": "single GPU"},
        "stages_ms": {"quantize": round(t_q, 4), "gemm": round(t_g, 4)},
        "roofline": {
            "kernel": "k5_gemm (block-scaled INT8 product)",
            "bound": "mfma",
            "achieved": round(gemm_tops, 1),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOPS (INT8)",
            "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
            "traffic": read_counters(W8A8_COUNTERS, W8A8_SOURCE) if name == "wan14b-720p-proj" else None,
            "avg_launch_ms": round(t_g, 4),
            "ops_i8_per_launch": ops,
        },
    }
    if not args.no_cpu_baseline:
        del ws, x8, xs
        result["cpu_baseline"] = cpu_baseline_w8a8(x, w, bias, wl, rows=1024)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def main_backward(args):
    """The SLA backward for the forward's own selection on the 720P pair: a step is one sagesla_backward."""
    import torch
    import int8_block_sparse_amd as sg
    import synth

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    sg.load()
    dev = torch.device("cuda:0")
    wl = synth.workload(WORKLOAD)
    log(f"generating {wl.name} inputs on the GPU")
    q, k, v, w = synth.make(wl, 0, device=dev)
    norm = None
    if args.qk_norm:
        gq, gk = synth.make_norm_weights(wl.H, wl.D, 0, device=dev)
        norm = (gq, gk, synth.NORM_EPS)
    _, ex = sg.forward(q, k, v, w, topk=wl.topk, export=True, norm=norm)
    mask = ex["block_idx"][..., :wl.topk].contiguous()
    del ex
    dy = torch.randn(q.shape, device=dev, generator=torch.Generator(device=dev).manual_seed(1)).to(torch.bfloat16)
    cfg = sg.Config(wl.B, wl.H, wl.N, wl.D, wl.blk_q, wl.blk_k, wl.topk, wl.linear, True, 0.0, False,
                    norm is not None)
    import ctypes
    pw = cfg.params(w_proj=w.data_ptr(), **sg._norm_args(norm, wl.H, wl.D))
    ws = torch.empty(sg.load().sagesla_backward_workspace_bytes(ctypes.byref(pw)), dtype=torch.uint8, device=dev)
    step = lambda: sg.backward(q, k, v, w, dy, mask, topk=wl.topk, workspace=ws, norm=norm)
    for _ in range(args.warmup):
        step()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(args.steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_ev = ev[0].elapsed_time(ev[1]) / args.steps
    log(f"{ms:.3f} ms per backward (events {ms_ev:.3f})")
    # algorithmic bf16 work of the sparse branch: S, dP, dV, dK, dQ per selected block pair (2 bq bk D each)
    pairs = wl.B * wl.H * wl.n_qb * wl.topk
    flops = pairs * 5 * 2.0 * wl.blk_q * wl.blk_k * wl.D
    tflops = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "SLA backward ms/layer (fixed selection), sparse-branch bf16 TFLOP/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s (5 products of 2*bq*bk*D per selected block pair)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16+f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D, "blk_q": wl.blk_q,
                   "blk_k": wl.blk_k, "topk": wl.topk, "linear": wl.linear, "qk_norm": bool(args.qk_norm),
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "sagesla_backward (all kernels)", "bound": "mfma", "achieved": round(tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s (bf16)", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "avg_launch_ms": round(ms_ev, 4), "flops_per_step": flops},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_backward(q, k, v, w, dy, mask, wl)
    print(json.dumps(result), flush=True)


def main_mfma_peak(args):
    """Practical matrix-core peak: a loop of independent MFMAs (no memory traffic) on every CU, timed with events;
    the clock the box holds under that load is what separates it from the published peaks."""
    import ctypes
    import torch

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    path = os.path.join(ROOT, "int8_block_sparse_amd", "libsagesla_probe.so")
    if not os.path.exists(path):
        sys.exit(f"{path} is missing: build it with `python -m int8_block_sparse_amd.build`")
    lib = ctypes.CDLL(path)
    lib.sagesla_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.sagesla_probe_mfma.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    blocks, iters = 256 * 8, 4096  # 8 workgroups of 4 waves per CU: 8 waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    kinds = {0: ("int8 v_mfma_i32_32x32x32_i8", 65536.0, PEAK_INT8_TOPS),
             1: ("bf16 v_mfma_f32_32x32x16_bf16", 32768.0, PEAK_BF16_TFLOPS),
             2: ("fp16 v_mfma_f32_32x32x16_f16", 32768.0, PEAK_BF16_TFLOPS)}
    res = {}
    for kind, (name, ops_each, peak) in kinds.items():
        for _ in range(max(1, args.warmup)):
            assert lib.sagesla_probe_mfma(kind, blocks, iters, 1, out.data_ptr(), stream) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            assert lib.sagesla_probe_mfma(kind, blocks, iters, i + 2, out.data_ptr(), stream) == 0
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        ops = blocks * 4 * 4.0 * iters * ops_each  # 4 waves x 4 MFMAs per iteration
        t = ops / (ms * 1e-3) / 1e12
        # the MFMA pipe needs 32 cycles per 32x32 op of these shapes on each SIMD (1024 SIMDs): the clock it held
        ghz = ops / ops_each * 32.0 / 1024 / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "achieved": round(t, 1), "peak": peak, "frac": round(t / peak, 4),
                     "implied_clock_ghz": round(ghz, 3)}
        log(f"{name}: {t:.1f} T/s ({t / peak:.3f} of {peak:.0f}), implied clock {ghz:.3f} GHz")
    name0 = kinds[0][0]
    print(json.dumps({"metric": "practical MFMA peak (independent MFMA loop, no memory)", "value": res[name0]["achieved"],
                      "unit": "TOPS (INT8)", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": res[name0]["ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                      "dtype": "i8", "data": "synthetic",
                      "config": {"workload": "mfma-peak", "workgroups": blocks, "iters": iters}, "kinds": res,
                      "cpu_baseline": None}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM-counter calibration under rocprofv3)")
    ap.add_argument("--qk-norm", action="store_true",
                    help="with the RMSNorm of Q and K before the path (sagesla and sla-backward workloads)")
    ap.add_argument("--workload", default="sagesla",
                    help="sagesla (the headline attention layer, wan14b-720p-sla-pair), another forward workload of "
                         "the synth module by name (tiny, wan1.3b-480p-dense, wan1.3b-480p-sla, 1080p-long-sla), "
                         "sla-backward (the headline layer's backward for the forward's selection) or w8a8-<shape> "
                         "(the W8A8 linear layer)")
    ap.add_argument("--summarize", choices=["trace", "hbm", "pmc"],
                    help="print a summary of rocprofv3 csv output instead of benchmarking: trace DIR (kernel-trace "
                         "stats), hbm FETCH_DIR WRITE_DIR (copy-calibrated FETCH_SIZE / WRITE_SIZE per kernel; with "
                         "--trace DIR the kernel-trace times beside them), pmc DIR... (counters averaged per kernel)")
    ap.add_argument("dirs", nargs="*", help="rocprofv3 output directories for --summarize")
    ap.add_argument("--trace", help="kernel-trace output directory (--summarize hbm / pmc)")
    ap.add_argument("--header", action="append", default=[], help="header line of the summary (repeatable)")
    ap.add_argument("--kernels", default="", help="--summarize pmc: comma-separated kernel name prefixes to keep")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the forward shards by "
              f"(batch, head) with no exchange, so N GPUs would each run this same kernel set on B*H/N heads.",
              file=sys.stderr)
        sys.exit(2)
    if args.workload.startswith("w8a8-"):
        return main_w8a8(args, args.workload[len("w8a8-"):])
    if args.workload == "sla-backward":
        return main_backward(args)
    if args.workload == "mfma-peak":
        return main_mfma_peak(args)
    import synth
    by_name = {w.name: w for w in synth.WORKLOADS.values()}
    name = HEADLINE if args.workload == "sagesla" else args.workload
    if name not in by_name:
        sys.exit(f"unknown workload {args.workload}; one of sagesla, sla-backward, w8a8-<shape>, "
                 f"{', '.join(sorted(by_name))}")
    return main_forward(args, by_name[name])


# ---------------------------------------------------------------------------------------------------------------
# summaries of rocprofv3 csv output (the tables committed under profiles/)
# ---------------------------------------------------------------------------------------------------------------
def _short_kernel(name):
    """'void sagesla::k3_attn<4, false>(signed char const*, ...)' -> 'k3_attn<4, false>'; other kernels keep a
    shortened name"""
    n = name.replace("void ", "", 1)
    if "sagesla::" in n:
        n = n.split("sagesla::", 1)[1]
        depth, cut = 0, len(n)
        for i, ch in enumerate(n):
            if ch == "<":
                depth += 1
            elif ch == ">":
                depth -= 1
            elif ch == "(" and depth == 0:
                cut = i
                break
        return n[:cut]
    return "torch " + n.split("(")[0][:40]


def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        sys.exit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _trace_ms(d):
    """average launch time (ms) and calls per kernel from a kernel-trace stats csv"""
    return {_short_kernel(r["Name"]): (float(r["AverageNs"]) * 1e-6, int(r["Calls"]))
            for r in _csv_rows(d, "kernel_stats.csv")}


def _counters(dirs):
    """per kernel and counter, the values of every dispatch"""
    acc = {}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            acc.setdefault(_short_kernel(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    return acc


def summarize(args):
    out = [f"# {h}" for h in args.header]
    if args.summarize == "trace":
        t = _trace_ms(args.dirs[0])
        total = sum(ms * c for ms, c in t.values())
        ours = {k: v for k, v in t.items() if not k.startswith("torch ")}
        out.append(f"{'kernel':40s} {'calls':>6s} {'avg_ms':>10s} {'share':>7s}")
        for k, (ms, c) in sorted(ours.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
            out.append(f"{k:40s} {c:6d} {ms:10.4f} {100 * ms * c / total:6.1f}%")
        other = [(ms, c) for k, (ms, c) in t.items() if k.startswith("torch ")]
        if other:
            out.append(f"{'torch kernels (seeded inputs, copies)':40s} {sum(c for _, c in other):6d} {'':>10s} "
                       f"{100 * sum(ms * c for ms, c in other) / total:6.1f}%")
    elif args.summarize == "hbm":
        f_dir, w_dir = args.dirs[:2]
        fetch = {k: v["FETCH_SIZE"] for k, v in _counters([f_dir]).items() if "FETCH_SIZE" in v}
        write = {k: v["WRITE_SIZE"] for k, v in _counters([w_dir]).items() if "WRITE_SIZE" in v}
        copy = [k for k in fetch if "copyBuffer" in k]
        if not copy or not args.calib_copy_mib:
            sys.exit("--summarize hbm needs the calibration copy (--calib-copy-mib M, as in the profiled run)")
        kib = args.calib_copy_mib * 1024.0
        f_scale, w_scale = kib / fetch[copy[0]][-1], kib / write[copy[0]][-1]
        out.append(f"# calibration: one {args.calib_copy_mib} MiB device copy reads FETCH_SIZE "
                   f"{fetch[copy[0]][-1]:.1f} KiB and WRITE_SIZE {write[copy[0]][-1]:.1f} KiB -> scale factors "
                   f"fetch {f_scale:.3f}, write {w_scale:.3f}")
        out.append("# bytes past L2 (served by the Infinity Cache or HBM) per kernel, averaged over its dispatches")
        tm = _trace_ms(args.trace) if args.trace else {}
        out.append(f"{'kernel':40s} {'fetch_GB':>10s} {'write_GB':>10s} {'avg_ms':>9s} {'GB/s':>9s}")
        per = {}
        for k in sorted(fetch, key=lambda k: -sum(fetch[k]) / len(fetch[k])):
            if k in copy or k not in write or k.startswith("torch "):
                continue
            fb = sum(fetch[k]) / len(fetch[k]) * f_scale * 1024
            wb = sum(write[k]) / len(write[k]) * w_scale * 1024
            per[k] = fb + wb
            ms = tm.get(k, (float("nan"), 0))[0]
            out.append(f"{k:40s} {fb / 1e9:10.3f} {wb / 1e9:10.3f} {ms:9.4f} {per[k] / ms / 1e6:9.1f}")
        out.append("")
        srcs = sorted({src for kern, src in HBM_KERNELS.items() if kern in per})
        for src in srcs:
            out.append(f"{src} sha256[:16]: {source_sha(os.path.join(CSRC, src))}")
        for kern in HBM_KERNELS:
            if kern in per:
                out.append(f"{kern} hbm bytes per launch (fetch+write, copy-calibrated): {per[kern]:.6g}")
                if kern in tm:
                    out.append(f"{kern} average launch (kernel trace) ms: {tm[kern][0]:.4f}")
        dom = max((k for k in per if k in HBM_KERNELS), key=lambda k: tm.get(k, (0, 0))[0], default=None)
        if dom:
            out.append(f"hbm bytes per launch (fetch+write, copy-calibrated): {per[dom]:.6g}")
    else:
        acc = _counters(args.dirs)
        tm = _trace_ms(args.trace) if args.trace else {}
        keep = [x for x in args.kernels.split(",") if x]
        for k, cs in sorted(acc.items()):
            if k.startswith("torch ") or (keep and not k.startswith(tuple(keep))):
                continue
            out.append(k + (f"   (kernel trace {tm[k][0]:.4f} ms)" if k in tm else ""))
            avg = {c: sum(v) / len(v) for c, v in cs.items()}
            for c in sorted(avg):
                out.append(f"   {c:32s} {avg[c]:16.6g}")
            if "GRBM_GUI_ACTIVE" in avg:
                cyc = avg["GRBM_GUI_ACTIVE"] / 8  # per XCD
                simd = 1024 * cyc
                if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                    out.append(f"{k} MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)): "
                               f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / simd:.4f}")
                if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
                    out.append(f"{k} VALU-MFMA co-execution fraction of SIMD cycles: "
                               f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / simd:.4f}")
                if "SQ_ACTIVE_INST_VALU" in avg:
                    out.append(f"{k} VALU active fraction of SIMD cycles (SQ_ACTIVE_INST_VALU x 4): "
                               f"{4 * avg['SQ_ACTIVE_INST_VALU'] / simd:.4f}")
                if "SQ_LDS_IDX_ACTIVE" in avg:
                    out.append(f"{k} LDS active fraction of CU cycles (SQ_LDS_IDX_ACTIVE / (256 x cycles)): "
                               f"{avg['SQ_LDS_IDX_ACTIVE'] / (256 * cyc):.4f}")
                if k in tm:
                    out.append(f"{k} shader clock implied over the launch: {cyc / tm[k][0] / 1e6:.3f} GHz")
            if "SQ_WAIT_ANY" in avg and "SQ_WAVE_CYCLES" in avg:
                out.append(f"{k} waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES): {avg['SQ_WAIT_ANY'] / avg['SQ_WAVE_CYCLES']:.4f}")
            for key, mul, what in (("SQ_INSTS_VALU_MFMA_MOPS_I8", 512, "INT8 MFMA ops per launch"),
                                   ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 512, "BF16 MFMA flops per launch"),
                                   ("SQ_INSTS_VALU_MFMA_MOPS_F16", 512, "FP16 MFMA flops per launch")):
                if key in avg:
                    out.append(f"{k} {what} ({key} x {mul}): {avg[key] * mul:.6g}")
        srcs = sorted({src for kern, src in HBM_KERNELS.items() if kern in acc})
        for src in srcs:
            out.append(f"{src} sha256[:16]: {source_sha(os.path.join(CSRC, src))}")
    print("\n".join(out))


def stage_bytes(wl):
    """Algorithmic HBM bytes of the quantize and linear stages of one forward: every input a kernel of the stage
    reads, once per kernel that reads it, and every output it writes (an intermediate that a later kernel of
    the stage consumes counts once written and once read). Layouts as the kernels store them."""
    BH, N, D, nqb, nkb = wl.B * wl.H, wl.N, wl.D, wl.n_qb, wl.n_kb
    bf16 = 2 * BH * N * D  # one bf16 [B][H][N][D] tensor
    lin_on = wl.linear and wl.topk < nkb
    quant = {
        "k1_colsum_partial": bf16,  # reads K
        "k1_quant": 3 * bf16  # reads Q, K, V
        + 2 * BH * N * D  # writes the INT8 codes of Q and K
        + BH * nkb * 16384  # V^T images of every key block (the tail block padded)
        + 4 * BH * (nqb + nkb) + 8 * BH * D * (nqb + nkb)  # scales, pooled means (fp64)
        + (BH * nkb * STATE_BYTES_PER_BLOCK if lin_on else 0),  # the linear branch's state table
    }
    lin = {}
    if lin_on:
        lin = {
            "k4_mask": 4 * BH * nqb * wl.topk + BH * nqb * ((nkb + 31) // 32) * 4,
            "k4_gemm16": BH * nkb * STATE_BYTES_PER_BLOCK + BH * nqb * REMAINING_BYTES_PER_QBLOCK,
        }
    return {"quantize": quant, "linear": lin}


def main_forward(args, wl):
    """One whole forward per step on a seeded workload of the synth module."""
    import torch
    import int8_block_sparse_amd as sg
    import synth

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    sg.load()
    dev = torch.device("cuda:0")
    log(f"generating {wl.name} inputs on the GPU")
    q, k, v, w = synth.make(wl, 0, device=dev)
    out = torch.empty_like(q)
    cfg = sg.Config(wl.B, wl.H, wl.N, wl.D, wl.blk_q, wl.blk_k, wl.topk, wl.linear)
    norm = None
    if args.qk_norm:
        gq, gk = synth.make_norm_weights(wl.H, wl.D, 0, device=dev)
        norm = (gq, gk, synth.NORM_EPS)
        cfg.qk_norm = True
    ws = torch.empty(sg.workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    fwd = lambda ev=None: sg.forward(q, k, v, w, topk=wl.topk, blk_q=wl.blk_q, blk_k=wl.blk_k, linear=wl.linear,
                                     out=out, workspace=ws, events=ev, norm=norm)
    for _ in range(args.warmup):
        fwd()
    evs = [sg.stage_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fwd(evs[i])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    stages = [sg.stage_ms(e) for e in evs]
    st_avg = {name: sum(s[name] for s in stages) / len(stages) for name in sg.STAGES}
    log(f"{ms:.3f} ms/layer; stages (ms): " + ", ".join(f"{n} {t:.3f}" for n, t in st_avg.items()))

    # cold variant: before each forward a 512 MiB device fill (twice the Infinity Cache) evicts the inputs and
    # intermediates from every cache; only the forward is timed (events on the current stream)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(args.steps):
        scrub.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fwd()
        e1.record()
        cold.append((e0, e1))
    torch.cuda.synchronize()
    cold_ms = sorted(a.elapsed_time(b) for a, b in cold)
    cold_med = cold_ms[len(cold_ms) // 2]
    del scrub
    log(f"cold (caches scrubbed before each forward): median {cold_med:.3f} ms/layer")

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    # roofline of the dominant kernel: the block-sparse attention (one launch = the attn stage). Algorithmic
    # work: per selected (query block, key block) pair S = Q K^T (INT8) and O = P V (bf16), 2 bq bk D each; per
    # query block of the linear branch phi(Q) H_m and (.) W_p, 2 bq D D bf16 each. The kernel also executes the
    # low-half products that carry the linear branch's bf16 operands to ~16 bits: counted apart, not in frac.
    units = wl.B * wl.H * wl.n_qb * wl.topk  # selected (query block, key block) pairs
    ops_i8 = units * 2.0 * wl.blk_q * wl.blk_k * wl.D
    ops_bf16 = units * 2.0 * wl.blk_q * wl.blk_k * wl.D
    lin_on = wl.linear and wl.topk < wl.n_kb
    epi = wl.B * wl.H * wl.n_qb * 2.0 * wl.blk_q * wl.D * wl.D  # one bq x D x D product per query block
    exec_bf16 = ops_bf16
    if lin_on:
        ops_bf16 += 2 * epi
        exec_bf16 += EPILOGUE_PRODUCTS_EXECUTED * epi
    t_attn = st_avg["attn"] * 1e-3
    int8_equiv = (ops_i8 + ops_bf16 * PEAK_INT8_TOPS / PEAK_BF16_TFLOPS) / t_attn / 1e12
    exec_equiv = (ops_i8 + exec_bf16 * PEAK_INT8_TOPS / PEAK_BF16_TFLOPS) / t_attn / 1e12
    headline = wl.name == HEADLINE
    traffic = read_counters() if headline else None
    dense_tops = wl.dense_equiv_ops / (ms * 1e-3) / 1e12
    # achieved algorithmic HBM bandwidth of the bandwidth-bound stages, live (the stage events bracket them)
    sb = stage_bytes(wl)
    hbm = {}
    for st, kern in sb.items():
        if not kern:
            continue
        byt = float(sum(kern.values()))
        t = st_avg[st] * 1e-3
        hbm[st] = {"kernels": sorted(kern), "algorithmic_bytes": byt, "ms": round(st_avg[st], 4),
                   "achieved_GBps": round(byt / t / 1e9, 1), "peak_GBps": PEAK_HBM_GBPS,
                   "frac": round(byt / t / 1e9 / PEAK_HBM_GBPS, 4)}
    metric = METRIC if headline else (f"SageSLA fwd ms/layer + dense-equiv TOPS (% INT8 MFMA peak), N={wl.N} "
                                      f"H={wl.H} D={wl.D}")
    result = {
        "metric": metric,
        "value": round(dense_tops, 2),
        "unit": "TOPS (dense-equivalent, 4*B*H*N^2*D per layer)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D,
                   "grid": list(wl.grid) if wl.grid else None, "structured": wl.structured,
                   "blk_q": wl.blk_q, "blk_k": wl.blk_k, "topk_frac": wl.topk_frac, "topk": wl.topk,
                   "linear": wl.linear, "qk_norm": bool(args.qk_norm), "parallelism": "single GPU"},
        "stages_ms": {n: round(t, 4) for n, t in st_avg.items()},
        "cold_ms_per_step": round(cold_med, 4),
        "roofline": {
            "kernel": "k3_attn (block-sparse INT8 attention" + (" + linear-branch epilogue)" if lin_on else ")"),
            "bound": "mfma",
            "achieved": round(int8_equiv, 1),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOPS (INT8-equivalent: INT8 ops + 2x BF16 flops)",
            "frac": round(int8_equiv / PEAK_INT8_TOPS, 4),
            "traffic": traffic,
            "mfma_util_at_box_clock": read_mfma_util() if headline else None,
            "avg_launch_ms": round(st_avg["attn"], 4),
            "ops_i8_per_launch": ops_i8,
            "flops_bf16_per_launch": ops_bf16,
            "executed_flops_bf16_per_launch": exec_bf16,
            "executed_frac": round(exec_equiv / PEAK_INT8_TOPS, 4),
        },
        "hbm_stages": hbm,
    }
    if headline:
        # per kernel, from the committed counter summary of the same sources: HBM bytes past L2 (FETCH_SIZE +
        # WRITE_SIZE, copy-calibrated) over the kernel-trace launch time, beside the algorithmic bytes
        kern = read_kernel_hbm()
        alg = {**sb["quantize"], **sb["linear"]}
        for name, d in kern.items():
            base = name.split("<")[0]
            if base in alg:
                d["algorithmic_bytes"] = float(alg[base])
                d["algorithmic_frac"] = round(alg[base] / d["ms"] / 1e6 / PEAK_HBM_GBPS, 4)
        result["hbm_kernels_profiled"] = kern
    if not args.no_cpu_baseline:
        # a bounded sample of whole (b, h) heads, about 10-30 s of CPU work
        del ws
        heads = [(0, 0), (wl.B - 1, wl.H - 1)] + [(b, h) for b in range(wl.B) for h in range(wl.H)]
        heads = list(dict.fromkeys(heads))[:CPU_HEADS.get(wl.name, 2)]
        gpu_sel = None
        if 0 < wl.topk < wl.n_kb:
            # one more forward (untimed) exporting the selection, checked against the oracle's on the same heads
            _, ex = sg.forward(q, k, v, w, topk=wl.topk, blk_q=wl.blk_q, linear=wl.linear, export=True)
            torch.cuda.synchronize()
            gpu_sel = {(b, h): (ex["scores"][b, h].cpu().numpy(), ex["block_idx"][b, h].cpu().numpy())
                       for (b, h) in heads}
            del ex
        cb = cpu_baseline(q, k, v, w, wl, heads, budget_s=20.0, blocks=CPU_BLOCKS.get(wl.name), gpu_sel=gpu_sel)
        if "selection_check" in cb:
            result["selection_check"] = cb.pop("selection_check")
        result["cpu_baseline"] = cb
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
