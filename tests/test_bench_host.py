"""Host-side pieces of bench.py (CPU only): the committed counter summaries parse, and a summary taken on
another kernel source is ignored."""
import os

import bench


def test_counter_summary_parses(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("// kernel\n")
    sha = bench.source_sha(str(src))
    f = tmp_path / "c.txt"
    f.write_text("# header: with a colon\nkernel   1.0   2.0\n\n"
                 f"k.hip sha256[:16]: {sha}\nFETCH_SIZE KiB per launch: 10.0\n"
                 "hbm bytes per launch (fetch+write, copy-calibrated): 1.5e+09\n")
    assert bench.read_counters(str(f), str(src)) == 1.5e9
    src.write_text("// changed kernel\n")
    assert bench.read_counters(str(f), str(src)) is None


def test_committed_summaries_have_the_parsed_keys():
    for path, source in ((bench.COUNTERS, bench.K3_SOURCE), (bench.W8A8_COUNTERS, bench.W8A8_SOURCE)):
        assert os.path.exists(path)
        text = open(path).read()
        assert f"{os.path.basename(source)} sha256[:16]: " in text
        assert "hbm bytes per launch (fetch+write, copy-calibrated): " in text


def test_mfma_summary_parses_and_is_source_gated(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("// kernel\n")
    f = tmp_path / "m.txt"
    f.write_text(f"# a: b\nk.hip sha256[:16]: {bench.source_sha(str(src))}\n"
                 "k4_gemm16 MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)): 0.11\n"
                 "k3_attn<4, false> MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)): "
                 "0.5552\n")
    assert bench.read_mfma_util(str(f), str(src)) == 0.5552
    src.write_text("// changed kernel\n")
    assert bench.read_mfma_util(str(f), str(src)) is None
    u = bench.read_mfma_util()  # None once the kernel has changed since the committed summary was taken
    assert u is None or 0.0 < u <= 1.0


def test_stage_bytes_of_the_headline_layer():
    # quantize stage: K read by the column sums, Q K V read and codes + V^T images written by the quantizer, which
    # with the linear branch on also writes the fp16 state table (129 rows of 128 fp16 per 64-key block)
    import synth
    wl = synth.WORKLOADS[3]
    sb = bench.stage_bytes(wl)
    elems = wl.B * wl.H * wl.N * wl.D
    table = wl.B * wl.H * wl.n_kb * 129 * 128 * 2
    assert abs(sum(sb["quantize"].values()) - (12 * elems + table)) < 0.02 * 12 * elems
    assert set(sb["linear"]) == {"k4_mask", "k4_gemm16"}
    dense = synth.WORKLOADS[1]
    sd = bench.stage_bytes(dense)
    assert not sd["linear"]  # the dense layer runs no linear branch, and its quantizer writes no table
    de = dense.B * dense.H * dense.N * dense.D
    assert abs(sum(sd["quantize"].values()) - 12 * de) < 0.02 * 12 * de



def test_kernel_hbm_summary_parses_and_is_source_gated(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    for name in ("k_attn.hip", "k_quant.hip", "k_linear.hip"):
        (csrc / name).write_text(f"// {name}\n")
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    sha = {n: bench.source_sha(str(csrc / n)) for n in ("k_attn.hip", "k_quant.hip", "k_linear.hip")}
    f = tmp_path / "h.txt"
    f.write_text("# header: x\n" + "".join(f"{n} sha256[:16]: {s}\n" for n, s in sha.items())
                 + "k1_quant<128, false> hbm bytes per launch (fetch+write, copy-calibrated): 8e+09\n"
                 + "k1_quant<128, false> average launch (kernel trace) ms: 2.0\n"
                 + "k4_gemm16 hbm bytes per launch (fetch+write, copy-calibrated): 4e+09\n"
                 + "k4_gemm16 average launch (kernel trace) ms: 1.0\n")
    got = bench.read_kernel_hbm(str(f))
    assert got["k1_quant<128, false>"]["achieved_GBps"] == 4000.0 and got["k1_quant<128, false>"]["frac"] == 0.5
    assert got["k4_gemm16"]["frac"] == 0.5 and "k3_attn<4, false>" not in got
    (csrc / "k_linear.hip").write_text("// changed\n")
    assert set(bench.read_kernel_hbm(str(f))) == {"k1_quant<128, false>"}


def test_short_kernel_names():
    assert bench._short_kernel("void sagesla::k3_attn<4, false>(signed char const*, int)") == "k3_attn<4, false>"
    assert bench._short_kernel("sagesla::k4_gemm16(unsigned short const*, int)") == "k4_gemm16"
    assert bench._short_kernel("void at::native::foo<1>(int)").startswith("torch ")


def test_selection_check_counts_rows_and_score_bound():
    # the bench line's selection diagnostics on a tiny oracle head: the oracle's own scores and lists agree with
    # themselves, a changed list row is counted (and, with a wide gap, as not a near tie), and a score moved by
    # more than the rounding bound shows a ratio above 1
    import math
    import numpy as np
    import synth
    from oracle import sagesla as orc
    wl = synth.workload(0)
    q, k, v, w = synth.make(wl, 0)
    f = lambda t: t.float().double().numpy()
    r = orc.forward_head(f(q[0, 0]), f(k[0, 0]), f(v[0, 0]), f(w), wl.blk_q, wl.blk_k, wl.topk, linear=False)
    s = r["scores"] * math.sqrt(wl.D)
    c = bench.selection_check(r, s, r["idx"].copy(), wl.D)
    assert c["rows"] == wl.n_qb and c["rows_differ"] == 0 and c["max_diff_over_bound"] <= 1.0
    idx = r["idx"].copy()
    row = int(np.argmax(r["gap"] * (r["gap"] < np.inf)))  # a row with a clear gap
    idx[row, -1] = next(J for J in range(wl.n_kb) if J not in idx[row])
    s2 = s.copy()
    s2[0, 0] += 1e-6 * max(1.0, abs(s2[0, 0]))
    c = bench.selection_check(r, s2, idx, wl.D)
    assert c["rows_differ"] == 1 and c["rows_differ_not_near_tie"] == (1 if r["gap"][row] >= orc.NEAR_TIE else 0)
    assert c["max_diff_over_bound"] > 1.0
