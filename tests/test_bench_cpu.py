"""Host-side logic of bench.py (no GPU): the amd-smi readers of --power and the
gate that reports the committed HBM traffic only for unchanged kernel code."""

import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

# The layout `amd-smi metric -p -c` prints (power, then one block per clock
# domain); the readers must take the GFX domains' current clocks only.
METRIC_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1388 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 2300 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 2340 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 2000 MHz
            MIN_CLK: 2000 MHz
        VCLK_0:
            CLK: 59 MHz
"""

LIST_TEXT = """GPU: 0
    BDF: 0000:05:00.0
    UUID: aaaa
GPU: 1
    BDF: 0000:75:00.0
    UUID: bbbb
"""


def fake_run(text, seen=None):
    def run(cmd, **kw):
        if seen is not None:
            seen.append(cmd)
        return types.SimpleNamespace(stdout=text, returncode=0)
    return run


def test_smi_sample_reads_socket_power_and_gfx_clocks(monkeypatch):
    seen = []
    monkeypatch.setattr(subprocess, "run", fake_run(METRIC_TEXT, seen))
    power, clocks = bench.smi_sample(3)
    assert power == 1388.0
    assert clocks == [2300.0, 2340.0]           # not MEM_0 or VCLK_0, not MIN/MAX
    assert seen[0][:5] == ["amd-smi", "metric", "-g", "3", "-p"]


def test_smi_sample_without_readings_or_tool(monkeypatch):
    monkeypatch.setattr(subprocess, "run", fake_run("GPU: 0\n    POWER:\n        SOCKET_POWER: N/A\n"))
    assert bench.smi_sample(0) is None

    def missing(cmd, **kw):
        raise FileNotFoundError(cmd[0])
    monkeypatch.setattr(subprocess, "run", missing)
    assert bench.smi_sample(0) is None


def test_smi_gpu_matches_pci_bus(monkeypatch):
    import torch

    monkeypatch.setattr(subprocess, "run", fake_run(LIST_TEXT))
    monkeypatch.setattr(torch.cuda, "get_device_properties",
                        lambda dev: types.SimpleNamespace(pci_domain_id=0, pci_bus_id=0x75))
    assert bench.smi_gpu(0) == (1, "0000:75:00.0")
    monkeypatch.setattr(torch.cuda, "get_device_properties",
                        lambda dev: types.SimpleNamespace(pci_domain_id=0, pci_bus_id=0x99))
    assert bench.smi_gpu(0) == (None, None)     # no sensors read rather than another GPU's


def test_code_sha256_ignores_comments_and_spacing(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("/* doc */ int f(int x)\n{ return x + 1; }\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.code_sha256(str(a)) == bench.code_sha256(str(b))
    assert bench.code_sha256(str(a)) != bench.code_sha256(str(c))


def test_traffic_reported_only_for_the_recorded_code(monkeypatch, tmp_path):
    csrc = os.path.join(ROOT, "quantized_flash_attn_amd", "csrc")
    sums = {n: bench.code_sha256(os.path.join(csrc, n)) for n in bench.ATTN_SRCS}
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps({"sources_code_sha256": sums,
                               "kernels": {"attn_fwd_kernel": {"traffic_bytes": 12345}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.measured_traffic(3) == 12345
    assert bench.measured_traffic(2) is None     # counters were taken on workload 3 only
    rec.write_text(json.dumps({"sources_code_sha256": dict(sums, **{bench.ATTN_SRCS[0]: "0" * 64}),
                               "kernels": {"attn_fwd_kernel": {"traffic_bytes": 12345}}}))
    assert bench.measured_traffic(3) is None     # the kernel changed since


def test_committed_traffic_summary_is_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert set(bench.ATTN_SRCS) <= set(rec["sources_code_sha256"])
    attn = rec["kernels"]["attn_fwd_kernel"]
    # fetch and write scaled by the copy-kernel factors recorded beside them
    assert attn["traffic_bytes"] == attn["fetch_bytes"] + attn["write_bytes"]
    assert abs(attn["fetch_bytes"] - attn["fetch_kib_raw"] * 1024 * rec["fetch_factor"]) < 1024 * rec["fetch_factor"]
    assert abs(attn["write_bytes"] - attn["write_kib_raw"] * 1024 * rec["write_factor"]) < 1024 * rec["write_factor"]


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stdout


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-q"]))
