"""Host code under the compiler's sanitizers (CPU only, no GPU involved).

* The CPU oracle, built with AddressSanitizer and UndefinedBehaviorSanitizer
  (float-to-int overflow included), runs every function on random and
  special inputs (tests/sanitize/oracle_driver.c).
* The host half of the library -- plans, argument validation, the
  multi-tensor table, the host AdamW thread pool -- built with g++ against
  host stand-ins for the device code (tests/sanitize/host_stubs.cpp), runs
  tests/sanitize/host_driver.cpp under AddressSanitizer + UBSan, and its
  concurrent part under ThreadSanitizer.

Each program must exit 0 and print nothing from a sanitizer.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fsdp_sharded_mixed_flatten_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ASAN_UBSAN = ["-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc/g++")


def _build(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"build failed: {' '.join(cmd)}\n{res.stderr[-4000:]}"


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", TSAN_OPTIONS="halt_on_error=1")
    res = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, f"{os.path.basename(exe)} {args} exited {res.returncode}:\n{out[-6000:]}"
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer", "ERROR: LeakSanitizer"):
        assert marker not in out, out[-6000:]
    return out


def _host_sources():
    return [os.path.join(CSRC, "zs_api.cpp"), os.path.join(CSRC, "zs_host_adamw.cpp"),
            os.path.join(SAN, "host_stubs.cpp"), os.path.join(SAN, "host_driver.cpp")]


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _build(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", *ASAN_UBSAN,
            os.path.join(ROOT, "oracle", "zs_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-lpthread",
            "-o", exe])
    assert "oracle driver ok" in _run(exe)


@pytest.fixture(scope="module")
def host_asan(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("host") / "host_san")
    _build(["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-pthread", *ASAN_UBSAN,
            f"-I{os.path.join(ROOT, 'include')}", *_host_sources(), "-o", exe])
    return exe


def test_host_library_under_asan_ubsan(host_asan):
    assert "host driver ok (all)" in _run(host_asan, "all")


def test_call_trace(host_asan):
    """ZS_LOG=1: one stderr line per call that enqueues work, numbered in
    order, naming the entry point, world size, rank, contributions and range."""
    env = dict(os.environ, ZS_LOG="1")
    res = subprocess.run([host_asan, "all"], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    lines = [ln for ln in res.stderr.splitlines() if ln.startswith("zs ")]
    seqs = [int(ln.split()[1]) for ln in lines]
    assert seqs == list(range(1, len(seqs) + 1))
    ops = {ln.split()[2] for ln in lines}
    for op in ("zs_reduce_shard", "zs_fused_shard_step", "zs_fused_shard_step_dc", "zs_accumulate_shard",
               "zs_grad_stats", "zs_clip_scale", "zs_multi_bind", "zs_fused_shard_step_multi", "zs_multi_unbind"):
        assert op in ops, (op, sorted(ops))
    assert any("zs_reduce_shard world=4 rank=1 contribs=4 off=0" in ln for ln in lines)
    # off by default: no trace lines
    res = subprocess.run([host_asan, "all"], capture_output=True, text=True, timeout=600)
    assert not [ln for ln in res.stderr.splitlines() if ln.startswith("zs ")]


def test_host_library_under_tsan(tmp_path):
    exe = str(tmp_path / "host_tsan")
    # the thread sanitizer's runtime cannot resolve the host AdamW's per-ISA
    # variants at load time: build the baseline variant only
    _build(["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-pthread", "-fsanitize=thread",
            "-DZS_HOST_ONE_ISA", f"-I{os.path.join(ROOT, 'include')}", *_host_sources(), "-o", exe])
    assert "host driver ok (threads)" in _run(exe, "threads")
