"""Host-only tests of the resident expert table's state machine (csrc/table_core.h).

tests/table_cpu/table_sim.cpp drives the same C++ code the library runs, over a
simulated transport whose streams execute lazily (a missing wait becomes a
consumer reading overwritten bytes) and whose calls can be made to fail.  It is
built with g++ twice: with the address and undefined-behaviour sanitizers
(every scenario) and with the thread sanitizer (several tables on several
threads sharing the copy pool).  Scenarios: random decode steps against
consumer reads (consumer first or copies first), a consumer on the default
stream, speculative prefetch before each step, staging reuse after its copy retired, open leases holding rows
and maps, failures before publication (old generation intact and current),
a failure after publication (table faulted), create-time rejections (spare
rows, staging, digests, non-finite scales) and the source re-check.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "table_cpu", "table_sim.cpp")


def build(tmp_path, name, flags):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / name)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-fno-omit-frame-pointer", "-pthread", *flags, "-o", exe, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return exe


def run(exe, scenario, env_extra):
    env = dict(os.environ, **env_extra)
    res = subprocess.run([exe, scenario], capture_output=True, text=True, timeout=600, env=env)
    assert res.returncode == 0, f"{scenario}:\n{res.stdout}\n{res.stderr[-6000:]}"
    return res.stdout


def test_table_state_machine_asan_ubsan(tmp_path):
    exe = build(tmp_path, "table_sim_asan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"])
    out = run(exe, "all", {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"})
    for name in ("steps", "default_stream", "prefetch", "staging", "direct", "lease", "fail_before", "fail_after",
                 "create", "threads"):
        assert f"{name}: ok" in out


def test_table_copy_pool_tsan(tmp_path):
    exe = build(tmp_path, "table_sim_tsan", ["-fsanitize=thread"])
    out = run(exe, "threads", {"TSAN_OPTIONS": "halt_on_error=1:second_deadlock_stack=1"})
    assert "threads: ok" in out
