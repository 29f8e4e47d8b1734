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
                 "MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)): 0.5552\n")
    assert bench.read_mfma_util(str(f), str(src)) == 0.5552
    src.write_text("// changed kernel\n")
    assert bench.read_mfma_util(str(f), str(src)) is None
    u = bench.read_mfma_util()  # None once the kernel has changed since the committed summary was taken
    assert u is None or 0.0 < u <= 1.0


def test_stage_bytes_of_the_headline_layer():
    # quantize stage: K read by the column sums, Q K V read and codes + V^T images written by the quantizer
    import synth
    wl = synth.WORKLOADS[3]
    sb = bench.stage_bytes(wl)
    elems = wl.B * wl.H * wl.N * wl.D
    assert abs(sum(sb["quantize"].values()) - 12 * elems) < 0.02 * 12 * elems
    assert set(sb["linear"]) == {"k4_states", "k4_mask", "k4_gemm"}
    assert not bench.stage_bytes(synth.WORKLOADS[1])["linear"]  # the dense layer runs no linear branch

