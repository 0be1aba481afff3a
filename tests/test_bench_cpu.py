"""Host-side pieces of bench.py (no GPU needed): the lookup of the committed HBM counter
summary that fills the roofline's `traffic` field, and the refusal of more than one GPU."""
import os

import bench


def test_counter_traffic_reads_committed_summary():
    """The summary's byte counts are returned while its stored source digests match the
    sources, for both kernels it covers."""
    cases = {bench.TRAFFIC_FILE: (("project", "project.hip"), ("gather", "gather.hip"),
                                  ("gather_lds", "gather.hip"), ("gather_lds_uniform", "gather.hip")),
             bench.TRAFFIC_DECODE: (("decode_project", "project.hip"),
                                    ("draft_project", "project.hip")),
             bench.TRAFFIC_BASIC: (("basic_sum", "basic.hip"), ("basic_sum_uniform", "basic.hip"))}
    for path, kernels in cases.items():
        kv = {}
        for ln in open(path):
            if "hbm_bytes_per_launch" in ln and not ln.startswith("#"):
                name, val = ln.split(" hbm_bytes_per_launch: ")
                kv[name] = float(val)
        assert set(kv) == {k for k, _ in kernels}, path
        for kernel, src in kernels:
            stored = [ln.rsplit(": ", 1)[1].strip() for ln in open(path)
                      if ln.startswith(f"{src} sha256[:16]: ")]
            assert len(stored) == 1
            want = kv[kernel] if stored[0] == bench.source_digest(src) else None
            assert bench.counter_traffic(kernel, src, path) == want


def test_counter_traffic_rejects_other_source(tmp_path, monkeypatch):
    """A summary taken on a different source (digest mismatch) gives no traffic figure."""
    f = tmp_path / "traffic.txt"
    digest = bench.source_digest("gather.hip")
    f.write_text("# header: ignored\n"
                 f"gather.hip sha256[:16]: {digest}\n"
                 "project.hip sha256[:16]: 0000000000000000\n"
                 "project hbm_bytes_per_launch: 123\n"
                 "gather hbm_bytes_per_launch: 456.5\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.counter_traffic("gather", "gather.hip") == 456.5
    assert bench.counter_traffic("project", "project.hip") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", os.path.join(str(tmp_path), "missing.txt"))
    assert bench.counter_traffic("gather", "gather.hip") is None


def test_more_than_one_gpu_is_refused_before_any_device_work():
    """`--gpus N` with N > 1 exits with a message (status 2) and touches no device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""
