"""bench.py's command line on the host (no GPU): more than one GPU is refused with a
message before anything touches a device, and the fused launch's traffic constants are
tied to the kernel sources they were measured on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_constants_carry_a_source_hash():
    sys.path.insert(0, ROOT)
    import bench
    h = bench.kernel_src_hash()
    assert len(h) == 16 and all(ch in "0123456789abcdef" for ch in h)
    t = bench.FUSED_TRAFFIC
    assert set(t) == {"src_sha256_16", "fetch_bytes", "write_bytes"}
    if not t["src_sha256_16"]:
        return   # not measured for these sources: the bench reports traffic as null
    assert len(t["src_sha256_16"]) == 16
    # the calibrated bytes a fused launch moves: at least the rows it must read (every
    # draft-slot row pair and W2), at most the input tensors plus pass 2's re-reads
    B, k, V, R = 64, 5, 129280, 256
    by_design = 2 * V * 2 * B * k + 2.0 * R * V
    assert by_design <= t["fetch_bytes"] <= 1.5 * by_design
    assert 0 < t["write_bytes"] < 0.1 * by_design
