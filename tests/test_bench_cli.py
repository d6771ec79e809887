"""bench.py's command line on the CPU: it measures one GPU only, and asking
for more GPUs ends with a message before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_field_follows_the_committed_counters():
    """roofline.traffic comes from profiles/gemm_ffn_traffic.txt only while the
    GEMM source is the one the counters were taken on (its sha256); the bytes
    are FETCH_SIZE and WRITE_SIZE scaled by the plain device copy's readings."""
    import hashlib
    sys.path.insert(0, ROOT)
    import bench
    path = os.path.join(ROOT, "profiles", "gemm_ffn_traffic.txt")
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    src = os.path.join(ROOT, "rotation_quantized_dit_amd", "csrc", "gemm_i8.hip")
    current = hashlib.sha256(open(src, "rb").read()).hexdigest()
    got = bench.measured_traffic("gemm_swiglu_up")
    if kv["gemm_source_sha256"] != current:
        assert got is None
        return
    cb = float(kv["copy_bytes"])
    want = (float(kv["gemm_swiglu_up.fetch_kib"]) * cb / float(kv["copy_fetch_kib"])
            + float(kv["gemm_swiglu_up.write_kib"]) * cb / float(kv["copy_write_kib"]))
    assert abs(got - want) <= 1e-9 * want
    # the write side is the bf16 output h [32256, 14336] to within 1 %
    write = float(kv["gemm_swiglu_up.write_kib"]) * cb / float(kv["copy_write_kib"])
    assert abs(write / (32256 * 14336 * 2) - 1.0) < 0.01
