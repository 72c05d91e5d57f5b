"""bench.py host logic (CPU): the one-GPU guard and the traffic records."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_records_parse_and_name_their_sources(tmp_path, monkeypatch):
    recs = [dict(kv.split("=", 1) for kv in line.split()) for line in open(bench.TRAFFIC_FILE)
            if line.strip() and not line.startswith("#")]
    kernels = {r["kernel"] for r in recs}
    for k in ("attn_fwd_kernel<128,4,1,false>", "permute_rows_kernel<gather>", "permute_rows_kernel<transition>",
              "permute_rows_kernel<scatter>", "rope_rows_kernel", "text_mean_kernel"):
        assert k in kernels, k
    for r in recs:
        assert os.path.exists(os.path.join(ROOT, r["source"])), r["source"]
        assert len(r["sha256"]) == 64 and int(r["fetch_bytes"]) > 0 and int(r["write_bytes"]) > 0

    # a record is used only while its source still hashes to the recorded value
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    import hashlib
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    rec = tmp_path / "traffic.txt"
    rec.write_text(f"kernel=foo_kernel<1> source={src} sha256={sha} workload=w fetch_bytes=10 write_bytes=5\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    monkeypatch.setattr(bench, "ROOT", "/")
    assert bench.measured_traffic("foo_kernel", "w") == {"fetch_bytes": 10, "write_bytes": 5, "total_bytes": 15}
    assert bench.measured_traffic("foo_kernel", "other") is None
    src.write_text("kernel source, changed\n")
    assert bench.measured_traffic("foo_kernel", "w") is None


def test_mfma_probe_library_validates_before_launch():
    """libwinprobe.so (bench.py's MFMA-loop ceiling) is built beside the
    library and refuses bad arguments without touching a device (fake
    pointers, never dereferenced)."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "window_attention_amd",
                        "libwinprobe.so")
    assert os.path.exists(path), "build() writes libwinprobe.so"
    lib = ctypes.CDLL(path)
    f = lib.win_probe_mfma_loop
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    f.restype = ctypes.c_int
    S, O = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)
    assert f(None, 1024, O, 1, 4, None) == -1
    assert f(S, 1024, None, 1, 4, None) == -1
    assert f(S, 1020, O, 1, 4, None) == -1          # not a whole number of 8-element fragments
    assert f(S, 1024, O, 0, 4, None) == -1
    assert f(S, 1024, O, 1, 0, None) == -1
    assert f(ctypes.c_void_p(0x10008), 1024, O, 1, 4, None) == -1  # misaligned
