"""Host code under the compilers' sanitizers (no GPU).

* The schedule functions the main kernel evaluates per tile
  (csrc/tile_sched.h) built with g++ under AddressSanitizer and
  UndefinedBehaviorSanitizer (tests/sched_host_check.cpp): every schedule,
  mask, tile ratio, KV-tile count (prime and composite) and ring size, checked
  against the closed forms, for exactly-once coverage and for a total order per
  dQ tile, with no out-of-bounds access, overflow or other undefined behaviour.
* The CPU model of the ordered dQ hand-off (tests/protocol_model.cpp) built with
  ThreadSanitizer: the accumulator adds, ordered only by the flag protocol, are
  free of data races under every dispatch form, and the runs still end with
  the rank-order bits.
"""
import os
import subprocess

import pytest

from test_protocol_model import expected_bits, run_model

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "deterministic_attention_backward_fa_amd", "csrc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")


def _build(tmp, src, flags):
    exe = str(tmp / os.path.splitext(src)[0])
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-pthread"] + flags +
                   ["-I", CSRC, os.path.join(HERE, src), "-o", exe], check=True)
    return exe


def test_schedule_functions_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path, "sched_host_check.cpp",
                 ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"])
    r = subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ") and int(r.stdout.split()[1]) > 300
    assert "runtime error" not in r.stderr


@pytest.fixture(scope="module")
def tsan_model(tmp_path_factory):
    return _build(tmp_path_factory.mktemp("tsan"), "protocol_model.cpp", ["-fsanitize=thread"])


@pytest.mark.parametrize("cfg", [
    # (schedule, causal, n_kv, r, mode (0 ticket, 1 rings), G, rings, threads)
    ("serial_ascending", True, 4, 2, 0, 0, 0, 4),
    ("descending_q", True, 4, 2, 1, 2, 2, 4),
    ("shift", False, 8, 1, 1, 4, 2, 8),
    ("symmetric_shift", True, 8, 2, 1, 2, 2, 4),
])
def test_protocol_model_under_tsan(tsan_model, cfg):
    sched, causal, n_kv, r, mode, G, rings, threads = cfg
    snake = mode == 1 and causal and sched == "descending_q"
    for seed in (1, 2):
        status, bits, walks, _, n_q = run_model(tsan_model, sched, causal, n_kv, r, 2, mode, G, rings, snake,
                                                threads, seed, timeout_ms=60000)
        assert status == "OK", (cfg, seed)
        assert bits == expected_bits(walks, 2, n_q), (cfg, seed)
