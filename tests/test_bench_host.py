"""Host-side checks of bench.py: the one-GPU guard, the committed HBM traffic record being
current for the routing sources, the counter scaling arithmetic, and the algorithmic byte count.
CPU only."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(spec)
spec.loader.exec_module(bench)

from expert_dispatch_layout_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_committed_traffic_record_is_current():
    """The stored counter profile must belong to the routing sources as they are, or bench.py
    reports no traffic."""
    rec = json.load(open(bench.TRAFFIC_JSON))
    assert rec["source_sha256"] == bench.route_sources_sha256()
    assert bench.traffic_from_profile() == rec["bytes_per_launch"]


def test_route_bytes_closed_form():
    wl = synth.WORKLOADS["dsv3"]
    # fp32 logits, the bias, and ids + weights per slot
    assert bench.route_bytes(wl) == wl.N * wl.E * 4 + wl.E * 4 + wl.N * wl.K * 8


def test_record_traffic_scaling(tmp_path, monkeypatch):
    wl = synth.WORKLOADS["dsv3"]
    name = bench.route_kernel_name(wl).split("<")[0]
    route = "void mep::%s<8, false, 1, 2>(args)" % name
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    hdr = "Kernel_Name,Counter_Name,Counter_Value\n"
    fetch.write_text(hdr + '"%s",FETCH_SIZE,100\n"%s",FETCH_SIZE,300\n"%s",FETCH_SIZE,512\n"%s",FETCH_SIZE,2\n'
                     % (route, route, bench.COPY_KERNEL, bench.COPY_KERNEL))
    write.write_text(hdr + '"%s",WRITE_SIZE,40\n"%s",WRITE_SIZE,1024\n' % (route, bench.COPY_KERNEL))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "t.json"))
    bench.record_traffic(str(fetch), str(write), 1, wl)
    rec = json.load(open(tmp_path / "t.json"))
    # 1 MiB copied: the copy's largest fetch reads 512 KiB (factor 2), its write 1024 (factor 1)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["bytes_per_launch"] == 1024 * (200 * 2.0 + 40 * 1.0)
    assert rec["source_sha256"] == bench.route_sources_sha256()
