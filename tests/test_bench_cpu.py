"""Host logic of bench.py that needs no GPU."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_profile_record_hash_ignores_comments_only():
    src = 'int a = 1; // note "x"\n/* block\n comment */ const char* s = "// kept"; char c = \'"\';\n'
    out = bench.strip_c_comments(src)
    assert "note" not in out and "block" not in out
    assert '"// kept"' in out and "'\"'" in out and "int a = 1;" in out
    assert bench.strip_c_comments(src.replace("note", "other note")) == out
    assert bench.strip_c_comments(src.replace("a = 1", "a = 2")) != out


def test_code_lines_ignore_added_comment_lines():
    src = "int f(int x) {\n  return x + 1;  // one\n}\n"
    out = bench.code_lines(src)
    assert bench.code_lines("// new line\n" + src.replace("// one", "// one\n  // two\n\n")) == out
    assert bench.code_lines(src.replace("x + 1", "x + 2")) != out
    assert out == "int f(int x) {\n  return x + 1;\n}"


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 64 and h == bench.kernel_source_hash()


def test_counted_flops_and_tiles():
    assert bench.counted_flops(1, 32, 8192, 128, True) == 10 * 32 * 8192 ** 2 * 128 / 2
    plan = {"n_q": 128, "n_kv": 64, "block_q": 64, "block_kv": 128}
    assert bench.tiles_executed(plan, 1, 32, True) == 133120
    assert bench.tiles_executed(plan, 1, 32, False) == 32 * 128 * 64


def test_trace_gantt_marks_compute_waits_and_switches():
    import numpy as np

    from deterministic_attention_backward_fa_amd import trace

    recs = np.zeros((3, 8, 2), dtype=np.int64)
    # workgroup 0: K/V staged (6) at 0, tile top (0) at 10, dS ready (1) at 30, dQ done (2) at 40,
    # turn (3) at 90 (a wait), adds (4) at 95, tile end (5) at 100
    recs[0, :7, 0] = [1000, 1010, 1030, 1040, 1090, 1095, 1100]
    recs[0, :7, 1] = [6, 0, 1, 2, 3, 4, 5]
    # workgroup 2 has a different counter base and ends halfway: its row starts at its own first record
    recs[2, :3, 0] = [5000, 5010, 5050]
    recs[2, :3, 1] = [6, 0, 1]
    g = trace.gantt(recs, width=20).splitlines()
    assert len(g) == 2 and g[0].startswith("   0 |") and g[1].startswith("   2 |")
    row0, row2 = g[0].split("|")[1], g[1].split("|")[1]
    assert row0[0] == "e" and "w" in row0 and row0.index("w") > row0.index("#")
    assert row2[0] == "e" and row2.rstrip().endswith("#") and row2.endswith(" ")
