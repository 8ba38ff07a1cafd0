"""Host-side pieces of bench.py: the kernel code hash that decides whether
the counter-measured traffic still applies (comments and layout do not
count, any code change does) and the per-element byte counts of the
roofline."""
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_text_drops_comments_and_layout_only():
    src = 'int a = 1; // one\n/* block\n comment */ int  b =\n 2;\nconst char* s = "x // not a comment";\nchar c = \'/\';'
    assert bench.code_text(src) == 'int a = 1; int b = 2; const char* s = "x // not a comment"; char c = \'/\';'
    assert bench.code_text('x = "a\\" // b"; // c') == 'x = "a\\" // b";'


def test_kernel_hash_ignores_comments_but_not_code():
    path = os.path.join(ROOT, "fsdp_sharded_mixed_flatten_amd", "csrc", "zs_kernels.hip")
    src = open(path).read()
    text = bench.code_text(src)
    commented = src.replace("constexpr int kBlock = kBlockThreads;",
                            "// a note\nconstexpr int kBlock = kBlockThreads;  /* and another */")
    assert commented != src and bench.code_text(commented) == text
    assert bench.code_text(src.replace("kGroup = 8;", "kGroup = 16;")) != text
    assert len(bench.kernel_hash()) == 16


@pytest.mark.parametrize("N", [1, 4, 8, 64])
def test_bytes_per_element(N):
    assert bench.reduce_bpp(N) == 2 * N + 2
    assert bench.adamw_bpp() == 28
    assert bench.fused_bpp(N) == 2 * N + 26
    assert bench.unfused_bpp(N) == (2 * N + 2) + 28 + 4


def test_counter_traffic_only_for_the_measured_world_size():
    import synth
    stock = bench.workload(synth, "llama7b")
    assert bench.traffic_key(stock) == "llama7b"
    assert bench.traffic_key(stock, "_bucketed") == "llama7b_bucketed"
    assert bench.traffic_key(bench.workload(synth, "llama7b", stock.world)) == "llama7b"
    resized = bench.workload(synth, "llama7b", 48)
    assert resized.world == 48 and bench.traffic_key(resized) is None
    assert bench.read_traffic("k_fused", None) is None


@pytest.mark.parametrize("gpus", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(gpus):
    import subprocess
    import sys
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(gpus)],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""
