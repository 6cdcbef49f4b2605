"""Host-side checks of bench.py's command line (no GPU needed): it measures one GPU and
refuses a multi-GPU run with a message and exit status 2, and its traffic record is
only reported for the kernel source it was measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def test_traffic_record_follows_the_kernel_source(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert rec["read_bytes"] + rec["write_bytes"] == rec["bytes_per_launch"]
    # reported only while the kernel source hashes to the one the counters were taken on
    assert bench.traffic_record() in (None, rec["bytes_per_launch"])
    # a change to the kernel file or to a header whose device code it inlines
    for i, name in enumerate(("gemm_fwd.hip", "common.h")):
        other = tmp_path / name
        other.write_text("// another version\n")
        srcs = list(bench.KERNEL_SRCS)
        srcs[[os.path.basename(f) for f in srcs].index(name)] = str(other)
        monkeypatch.setattr(bench, "KERNEL_SRCS", srcs)
        assert bench.traffic_record() is None
