"""Host-side logic of bench.py (no GPU): the HBM traffic a bench line reports
comes from a committed counter summary only while that summary's source hash
matches the kernels' sources, so a kernel changed after its counters were
taken reports null instead of a stale figure."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def write(tmp_path, text):
    p = tmp_path / "summary.md"
    p.write_text(text)
    return str(p)


def test_figure_read_only_under_a_matching_hash(bench, tmp_path):
    path = write(tmp_path, "# counters\n\nsource_sha256: abc123\nhbm_bytes_per_launch: 1234\n"
                           "hbm_bytes_per_launch_out: 99\n")
    assert bench.committed_traffic(path, "abc123") == 1234.0
    assert bench.committed_traffic(path, "abc123", key="hbm_bytes_per_launch_out") == 99.0
    assert bench.committed_traffic(path, "abc124") is None            # sources changed
    assert bench.committed_traffic(path, "abc123", key="missing") is None
    assert bench.committed_traffic(str(tmp_path / "absent.md"), "abc123") is None


def test_digests_cover_each_kernels_sources(bench):
    # each digest changes with the bytes of the sources it names, and the three
    # kernel families hash different files
    d = {bench.source_digest(), bench.softmax_source_digest(), bench.projection_source_digest()}
    assert len(d) == 3 and all(len(x) == 64 for x in d)
    assert bench._digest(("la_device.h",)) != bench._digest(("la_device.h", "sm_api.hip"))


def test_committed_summaries_name_their_figures(bench):
    # every hash-gated summary under profiles/ carries a hash and its figure
    # lines, in the form the bench reads
    for path, keys in ((bench.TRAFFIC_FILE, ["hbm_bytes_per_launch"]),
                       (bench.SOFTMAX_TRAFFIC_FILE, ["hbm_bytes_per_launch"]),
                       (bench.PROJECTION_TRAFFIC_FILE, ["hbm_bytes_per_launch",
                                                        "hbm_bytes_per_launch_out"])):
        text = open(path).read()
        assert "source_sha256: " in text
        for k in keys:
            assert "\n%s: " % k in text


def test_code_text_drops_comments_and_blank_lines_only(bench):
    ct = bench.code_text
    assert ct("int a; // note\nint b; /* two\n lines */ int c;\n\n   \n") == "int a;\nint b;   int c;"
    # comment markers inside string and character literals are code
    assert ct('s = "a//b /*c*/"; // t') == 's = "a//b /*c*/";'
    assert ct("c = '\\''; // q") == "c = '\\'';"
    assert ct('p = "\\"//"; x') == 'p = "\\"//"; x'
    # a comment edit keeps the text; any code edit changes it
    base = "float f(float x) {\n    return x * 2.0f;  // double\n}\n"
    assert ct(base) == ct(base.replace("// double", "// twice the input\n\n"))
    assert ct(base) != ct(base.replace("2.0f", "3.0f"))
    assert ct(base) != ct(base.replace("x * 2", "x*2"))


def test_digest_ignores_comment_edits(bench, tmp_path, monkeypatch):
    src = tmp_path / "k.h"
    src.write_text("// header\n__device__ int g(int a) { return a + 1; }\n")
    monkeypatch.setattr(bench, "SOURCES", str(tmp_path))
    d0 = bench._digest(("k.h",))
    src.write_text("// header, reworded\n\n__device__ int g(int a) { return a + 1; }  /* note */\n")
    assert bench._digest(("k.h",)) == d0
    src.write_text("// header\n__device__ int g(int a) { return a + 2; }\n")
    assert bench._digest(("k.h",)) != d0
