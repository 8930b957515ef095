"""Host logic of bench.py (no GPU): argument checks, the algorithmic byte
counts the roofline divides by, and the rule that counter traffic is reported
only for the kernel source it was measured on."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bad_step_counts_are_refused():
    assert _run("--steps", "0").returncode == 2
    assert _run("--warmup", "-1").returncode == 2


def test_algorithmic_bytes_of_the_decode_launch():
    b = _bench()
    # int8 token in: packed W 4 MiB + per-tensor scale + token + sx + fp32 out
    assert b.gemv_bytes(1, 4096, 4096, False) == 4096 * 1024 + 4 + 4096 + 4 + 4 * 4096 == 4214792
    # bf16 token in, int8 token and sx written, then the same contraction
    assert b.fused_bytes(1, 4096, 4096, 2, False) == 2 * 4096 + 4096 * 1024 + 4 + 4096 + 4 + 16384
    assert b.fused_bytes(1, 4096, 4096, 2, False) == 4222984
    # per-row scales add 4 bytes per row
    assert b.gemv_bytes(1, 6912, 2560, True) - b.gemv_bytes(1, 6912, 2560, False) == 4 * 6912 - 4


def _profile(tmp_path, digest, traffic):
    p = tmp_path / "profile.md"
    p.write_text("# summary\n\n- traffic_bytes_per_launch: `%s`\n"
                 "- kernel_source_sha256_16: `%s`\n" % (traffic, digest))
    return str(p)


def test_counter_traffic_only_for_the_measured_source(tmp_path):
    b = _bench()
    b.PROFILE = _profile(tmp_path, b.source_digest(), 4400000)
    assert b.counter_traffic() == 4400000
    b.PROFILE = _profile(tmp_path, "0" * 16, 4400000)
    assert b.counter_traffic() is None
    b.PROFILE = _profile(tmp_path, b.source_digest(), "n/a")
    assert b.counter_traffic() is None
    b.PROFILE = str(tmp_path / "missing.md")
    assert b.counter_traffic() is None


def test_source_digest_covers_the_decode_kernel_sources():
    b = _bench()
    names = sorted(os.path.basename(f) for f in b.KERNEL_SOURCES)
    assert names == ["k_gemv.hip", "tq_device.hpp"]
    assert len(b.source_digest()) == 16 and b.source_digest() == b.source_digest()


def test_source_digest_ignores_comments_not_code(tmp_path):
    b = _bench()
    src = tmp_path / "k.hip"
    hdr = tmp_path / "d.hpp"
    hdr.write_text("inline int f(int x) { return x + 1; }\n")
    b.KERNEL_SOURCES = [str(src), str(hdr)]
    src.write_text("__global__ void k(int* p) {\n  p[0] = 1;  // store\n}\n")
    d0 = b.source_digest()
    src.write_text("/* a kernel */\n__global__ void k(int* p) {\n\n  p[0] = 1;   // the store\n}\n")
    assert b.source_digest() == d0
    src.write_text("__global__ void k(int* p) {\n  p[0] = 2;  // store\n}\n")
    assert b.source_digest() != d0
