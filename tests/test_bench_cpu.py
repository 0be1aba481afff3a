"""Host-side pieces of bench.py: the lookup of the committed HBM counter summary that fills
the roofline's `traffic` field (no GPU needed)."""
import os

import bench


def test_counter_traffic_reads_committed_summary():
    """The summary's byte counts are returned while its stored source digests match the
    sources, for both kernels it covers."""
    kv = {}
    for ln in open(bench.TRAFFIC_FILE):
        if ln.startswith(("project", "gather")) and "bytes_per_launch" in ln:
            name, val = ln.split(" hbm_bytes_per_launch: ")
            kv[name] = float(val)
    assert set(kv) == {"project", "gather"}
    for kernel, src in (("project", "project.hip"), ("gather", "gather.hip")):
        stored = [ln.rsplit(": ", 1)[1].strip() for ln in open(bench.TRAFFIC_FILE)
                  if ln.startswith(f"{src} sha256[:16]: ")]
        assert len(stored) == 1
        want = kv[kernel] if stored[0] == bench.source_digest(src) else None
        assert bench.counter_traffic(kernel, src) == want


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
