"""bench.py host logic on the CPU: its refusals (more than one GPU, --one-stream without --fused)
and the HBM-traffic report, which scales the gate/up kernel's FETCH_SIZE and WRITE_SIZE counters
(KiB per dispatch) by their readings on a 256 MiB device copy and ties the result to a digest of the
kernel's sources."""
import hashlib
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_one_stream_needs_the_one_call_layer():
    r = run("--one-stream")
    assert r.returncode == 2 and "--fused" in r.stderr


def write_counters(directory, rows):
    os.makedirs(os.path.join(directory, "host"), exist_ok=True)
    with open(os.path.join(directory, "host", "p_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (kernel, counter, value) in enumerate(rows):
            f.write(f'{i},"{kernel}",{counter},{value}\n')


def test_traffic_report_scales_by_the_copy_and_records_the_source_digest(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    gu = "void (anonymous namespace)::w4a16_ffn_kernel<true, 16, 1, false>(ffn::FfnArgs)"
    down = "void (anonymous namespace)::w4a16_ffn_kernel<false, 8, 1, false>(ffn::FfnArgs)"
    d = {n: str(tmp_path / n) for n in ("gu_fetch", "gu_write", "copy_fetch", "copy_write")}
    # the copy of 256 MiB reads back half its bytes in FETCH_SIZE and all of them in WRITE_SIZE
    write_counters(d["copy_fetch"], [(copy, "FETCH_SIZE", 131072.0), (copy, "FETCH_SIZE", 131072.0)])
    write_counters(d["copy_write"], [(copy, "WRITE_SIZE", 262144.0)])
    # two gate/up dispatches (their mean counts) and a down dispatch that must be ignored
    write_counters(d["gu_fetch"], [(gu, "FETCH_SIZE", 67000.0), (gu, "FETCH_SIZE", 68000.0),
                                   (down, "FETCH_SIZE", 1.0e9)])
    write_counters(d["gu_write"], [(gu, "WRITE_SIZE", 512.0), (down, "WRITE_SIZE", 1.0e9)])
    out = str(tmp_path / "traffic.json")
    r = run("--traffic-report", d["gu_fetch"], d["gu_write"], d["copy_fetch"], d["copy_write"], out)
    assert r.returncode == 0, r.stderr
    got = json.load(open(out))
    assert got["workload"] == "olmoe_T32"
    assert got["fetch_factor"] == 2.0 and got["write_factor"] == 1.0
    assert got["fetch_bytes"] == 67500.0 * 1024 * 2
    assert got["write_bytes"] == 512.0 * 1024
    assert got["bytes_per_launch"] == got["fetch_bytes"] + got["write_bytes"]
    h = hashlib.sha256()
    for f in ("expert_ffn.hip", "ffn_stream.h", "ffn_common.h", "moe_internal.h"):
        with open(os.path.join(ROOT, "w4a16_routed_expert_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    assert got["source_sha256"] == h.hexdigest()


def test_traffic_report_fails_without_records(tmp_path):
    empty = str(tmp_path / "empty")
    os.makedirs(empty)
    r = run("--traffic-report", empty, empty, empty, empty, str(tmp_path / "t.json"))
    assert r.returncode != 0 and "no " in r.stderr
