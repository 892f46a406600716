"""CPU tests of bench.py's host logic against numbers the pages print
(tests/golden/io_model_examples.json, each entry citing its source)."""

import json
import os

import pytest

import bench
from workloads import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "io_model_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_io_complexity_worked_example(golden):
    g = golden["fa_notes_3_5_worked_example"]
    assert bench.standard_accesses(g["N"], g["d"]) == g["standard_accesses"]
    assert bench.flash_accesses(g["N"], g["d"], g["M_elements"]) == \
        pytest.approx(g["flash_accesses"], abs=1e-9)
    ratio = g["standard_accesses"] / g["flash_accesses"]
    assert round(ratio, 1) == g["ratio_approx"]


def test_materialised_matrix_sizes(golden):
    cases = [golden["fa_notes_2_1_score_matrix"],
             *golden["fa_notes_3_3_s_and_p"],
             golden["s12_why_it_matters"],
             golden["s12_how_it_works_diagram"]]
    for c in cases:
        b = bench.score_matrix_bytes(c["N"], c["bytes_per_element"],
                                     c["matrices"], c["heads"])
        assert b == c["MiB"] * 2 ** 20, c["cite"]


def test_compulsory_bytes_and_flop_counts():
    w = WORKLOADS["gpt2_medium_causal_4k"]
    nd = 2 * 16 * 4096 * 64
    assert bench.compulsory_bytes(w, False) == 2 * 4 * nd + 8 * 2 * 16 * 4096
    assert bench.compulsory_bytes(w, True) == 2 * 8 * nd + 8 * 2 * 16 * 4096
    # 4 B H N^2 d, halved when causal; backward 2.5x
    assert w.fwd_flops() == 4 * 2 * 16 * 4096 ** 2 * 64 / 2
    assert w.bwd_flops() == 2.5 * w.fwd_flops()
    t = WORKLOADS["tiny_f32"]
    assert t.fwd_flops() == 4 * 256 ** 2 * 64


def test_bench_refuses_several_gpus():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_source_hash_ignores_comments_and_layout_only():
    a = "int f(int x) {  // first comment\n  return x + 1;  /* two */ }\n"
    b = "/* other words */ int f(int x) {\n\treturn x + 1; // changed\n}"
    c = "int f(int x) { return x + 2; }"
    assert bench.strip_c_comments(a) == bench.strip_c_comments(b)
    assert bench.strip_c_comments(a) != bench.strip_c_comments(c)
    # comment markers inside literals are code, not comments
    assert bench.strip_c_comments('s = "a // b"; t = \'/\';') == \
        's = "a // b"; t = \'/\';'
    h = bench.source_hash()
    assert len(h) == 16 and h == bench.source_hash()
