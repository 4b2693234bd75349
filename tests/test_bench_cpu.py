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


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 64 and h == bench.kernel_source_hash()


def test_counted_flops_and_tiles():
    assert bench.counted_flops(1, 32, 8192, 128, True) == 10 * 32 * 8192 ** 2 * 128 / 2
    plan = {"n_q": 128, "n_kv": 64, "block_q": 64, "block_kv": 128}
    assert bench.tiles_executed(plan, 1, 32, True) == 133120
    assert bench.tiles_executed(plan, 1, 32, False) == 32 * 128 * 64
