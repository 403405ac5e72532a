"""Host-side checks of the rocprofv3 summarizer (no GPU)."""
import csv
import os

from llama2_decoder_layer_amd import profiling as P

HDR = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HDR)
        for i, (name, grid, ctr, val) in enumerate(rows):
            w.writerow([i, i, grid, name, ctr, val])


def test_traffic_calibration_and_digest(tmp_path, monkeypatch):
    k = "void ll::gemm_dma_kernel<1, 2, 256, 256, 1, 8>(ll::ProjArgs)"
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    # copy of 1 MiB reads as 512 KiB fetched (scale 2) and 1024 KiB written (scale 1);
    # a small copy dispatch must not be taken as the calibration.
    _write(fetch, [(P.COPY_KERNEL, 64, "FETCH_SIZE", 3.0), (P.COPY_KERNEL, 4096, "FETCH_SIZE", 512.0),
                   (k, 100, "FETCH_SIZE", 1000.0), (k, 100, "FETCH_SIZE", 1200.0)])
    _write(write, [(P.COPY_KERNEL, 4096, "WRITE_SIZE", 1024.0), (k, 100, "WRITE_SIZE", 10.0)])
    text = P.traffic_summary(str(fetch), str(write), "gemm_gate_up", "wl", 1.0, "a", "b")
    monkeypatch.setattr(P, "PROFILES", str(tmp_path))
    with open(P.traffic_path("gemm_gate_up", "wl"), "w") as f:
        f.write(text)
    t = P.load_traffic("gemm_gate_up", "wl")
    assert abs(t["fetch_bytes"] - 1100.0 * 1024 * 2) < 1
    assert abs(t["write_bytes"] - 10.0 * 1024) < 1
    assert abs(t["bytes"] - t["fetch_bytes"] - t["write_bytes"]) < 2
    # a summary taken on other sources is not used
    with open(P.traffic_path("gemm_gate_up", "wl"), "w") as f:
        f.write(text.replace(P.sources_digest("gemm_gate_up"), "0" * 16))
    assert P.load_traffic("gemm_gate_up", "wl") is None
    assert P.load_traffic("gemm_gate_up", "other") is None


def test_committed_summaries_parse():
    d = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
    for f in os.listdir(d):
        if f.endswith("_traffic.md"):
            txt = open(os.path.join(d, f)).read()
            assert "traffic_bytes_per_launch:" in txt and "sources_sha256:" in txt, f
