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
