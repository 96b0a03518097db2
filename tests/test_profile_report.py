"""bench.py's rocprofv3 harness on the CPU: the reduction of a small committed
fixture of rocprofv3 CSV output (tests/golden/rocprof: a kernel-stats file,
the bench line of the traced run, and one file per counter pass, with round
numbers) into the profile summaries, and the shape of the passes it runs."""

import json
import os

import pytest

import bench

FIX = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rocprof")


def test_counter_reduction_and_copy_calibration(tmp_path):
    M = bench.profile_report(FIX, "long", tag="fixture", profiles_dir=str(tmp_path))
    # the 256 MiB calibration copy reads FETCH_SIZE = 131072 KiB (half) and
    # WRITE_SIZE = 262144 KiB: scales 2 and 1; the small upload copy is ignored
    assert M["_fetch_scale"] == pytest.approx(2.0) and M["_write_scale"] == pytest.approx(1.0)
    f = M["fwd_kernel"]
    assert f["read_bytes"] == pytest.approx((200000 + 210000) / 2 * 2 * 1024)
    assert f["write_bytes"] == pytest.approx(66560 * 1024)
    # 14.4e6 GRBM cycles over 8 XCDs in 1 ms: 1.8 GHz; 921.6e6 busy cycles of
    # 1024 SIMDs x 1.8e6: 50 %; 6e6 VALU incl. 1e6 MFMA: 5 VALU per MFMA
    assert f["clock_ghz"] == pytest.approx(1.8) and f["mfma_busy_pct"] == pytest.approx(50.0)
    assert f["valu_per_mfma"] == pytest.approx(5.0) and f["lds_per_mfma"] == pytest.approx(1.5)
    assert f["lds_conflict_pct"] == pytest.approx(1.0)
    k = M["bwd_kv_kernel"]
    assert k["read_bytes"] == pytest.approx(710000 * 2 * 1024) and k["write_bytes"] == pytest.approx(131072 * 1024)
    assert k["clock_ghz"] == pytest.approx(1.8) and k["mfma_busy_pct"] == pytest.approx(40.0)
    assert k["valu_per_mfma"] == pytest.approx(4.0) and k["lds_conflict_pct"] == 0.0
    # the summaries and the traffic entry for this workload
    trace = (tmp_path / "fixture_kernel_trace.md").read_text()
    assert "| bwd_kv_kernel | 20 | 2000.0 |" in trace and "trace average 2.0000 ms" in trace
    counters = (tmp_path / "fixture_counters.md").read_text()
    assert "| fwd_kernel | 400.4 | 65.0 | 1.80 | 50.0 | 37.5 | 5.00 | 1.50 | 1.0 |" in counters
    assert "--pmc FETCH_SIZE" in counters and "--calibrate-copy 256" in counters
    t = json.loads((tmp_path / "hbm_traffic.json").read_text())["workloads"]["long"]
    assert t["fwd_kernel"]["fetch_bytes"] == 410000 * 1024 and t["fwd_kernel"]["write_bytes"] == 66560 * 1024
    assert t["bwd_kv_kernel"]["sources_sha256"] == bench.kernel_sources_sha256("bwd_kv_kernel")


def test_traffic_is_read_back_only_for_current_sources(tmp_path, monkeypatch):
    bench.profile_report(FIX, "gpt2", tag="fixture", profiles_dir=str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "hbm_traffic.json"))
    assert bench.measured_traffic("fwd_kernel", "gpt2") == 410000 * 1024 + 66560 * 1024
    assert bench.measured_traffic("fwd_kernel", "long") is None          # another workload
    d = json.loads((tmp_path / "hbm_traffic.json").read_text())
    d["workloads"]["gpt2"]["fwd_kernel"]["sources_sha256"] = "0" * 64   # the kernel changed since
    (tmp_path / "hbm_traffic.json").write_text(json.dumps(d))
    assert bench.measured_traffic("fwd_kernel", "gpt2") is None


def test_profile_passes_respect_counter_limits():
    """One trace pass without counters, then counter passes of at most 8 SQ,
    2 GRBM and 4 TCC counters (FETCH_SIZE takes 3, WRITE_SIZE 2), none
    combined with a trace domain; the program follows '--' directly."""
    cmds = bench.profile_commands("long", 20, python="python")
    assert [n for n, _ in cmds] == ["trace", "fetch", "write", "sq1", "sq2"]
    for name, argv in cmds:
        i = argv.index("--")
        assert argv[i + 1] == "python"
        if name == "trace":
            assert "--pmc" not in argv and "--kernel-trace" in argv
            continue
        counters = argv[argv.index("--pmc") + 1:argv.index("--kernel-include-regex")]
        assert not {"--sys-trace", "-s", "--runtime-trace", "-r", "--kernel-trace"} & set(argv)
        assert sum(c.startswith("SQ_") for c in counters) <= 8
        assert sum(c.startswith("GRBM_") for c in counters) <= 2
        assert 3 * counters.count("FETCH_SIZE") + 2 * counters.count("WRITE_SIZE") <= 4


def test_io_ablation_reduction(tmp_path):
    """Per configuration: the mean of its dispatches' byte counters, scaled by
    the copy (fetch x2, write x1), against the kernel's own byte model."""
    path = bench.io_ablation_report(os.path.join(FIX + "_io"), profiles_dir=str(tmp_path))
    text = open(path).read()
    # config 1: fetch mean 2000 KiB x 2 = 3.9 MiB, write 512 KiB = 0.5 MiB; (3.9 + 0.5) / (4 + 1) = 0.88
    assert "| 2048 | 64 | 1 | 1.5000 | 0.0500 | 4.0 / 1.0 | 3.0 / 0.5 | 3.9 / 0.5 | 0.88 |" in text
    # config 2: fetch mean 5000 KiB x 2 = 9.8 MiB, write 1 MiB; 10.8 / 12 = 0.90
    assert "| 4096 | 64 | 1 | 6.0000 | 0.1000 | 10.0 / 2.0 | 8.0 / 1.0 | 9.8 / 1.0 | 0.90 |" in text
    assert "--profile-mode io-ablation" in text
    # the query-outer forward: the last 3 fwd_kernel dispatches per N (the
    # earlier workload's dispatch is not among them); fetch (256, 512, 768)
    # KiB -> mean 512 x 2 = 1.0 MiB, write 512 KiB = 0.5 MiB
    assert "| 2048 | 0.0500 | 1.0 / 0.5 | - |" in text
    assert "| 4096 | 0.1000 | 2.0 / 1.0 | - |" in text


@pytest.mark.parametrize("mode", ["io-ablation", "compare-standard"])
def test_profile_modes_run_the_ablations(mode):
    cmds = bench.profile_commands("long", 8, python="python", mode=mode)
    assert cmds[0][0] == "trace" and ("--" + mode) in cmds[0][1]
    for name, argv in cmds[1:]:
        assert argv[argv.index("--") + 1] == "python" and ("--" + mode) in argv
        counters = argv[argv.index("--pmc") + 1:argv.index("--kernel-include-regex")]
        assert 3 * counters.count("FETCH_SIZE") + 2 * counters.count("WRITE_SIZE") <= 4


def test_sweep_markdown(tmp_path, monkeypatch):
    """bench.py --sweep-md: one table row per sweep point, with the command
    and the same run's main line."""
    monkeypatch.setattr("sys.argv", ["bench.py", "--sweep", "--sweep-md", "out.md"])
    rows = [{"sweep": True, "B": 4, "H": 16, "N": 4096, "d": 128, "causal": True, "fwd_ms": 0.25, "bwd_ms": 0.75,
             "fwd_tflops": 900.0, "bwd_tflops": 700.0, "fwd_pct": 36.0, "bwd_pct": 28.0}]
    line = {"config": {"workload": "long: B=1 H=16"}, "value": 850.0, "fwd_pct_peak": 42.0, "bwd_pct_peak": 33.0}
    p = tmp_path / "s.md"
    bench.write_sweep_md(str(p), rows, line)
    text = p.read_text()
    assert "python bench.py --sweep --sweep-md out.md" in text
    assert "| 4096 | 4 | 128 | yes | 0.2500 | 0.7500 | 900.0 (36.0) | 700.0 (28.0) |" in text
    assert "workload long): 850.00 TFLOP/s" in text


AMD_SMI_SAMPLE = """GPU: 0
    POWER:
        SOCKET_POWER: 1339 W
        GFX_VOLTAGE: N/A
        THROTTLE_STATUS: N/A
    CLOCK:
        GFX_0:
            CLK: 1799 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1801 MHz
            MIN_CLK: 500 MHz
"""


def test_amd_smi_parse_and_power_table(tmp_path, monkeypatch):
    """bench.py --power: the socket power and GFX_0's clock from amd-smi's
    text (values it does not show are None), and the table it writes."""
    assert bench.parse_amd_smi(AMD_SMI_SAMPLE) == (1339.0, 1799.0)
    assert bench.parse_amd_smi("GPU: 0\n    POWER:\n        SOCKET_POWER: N/A\n") == (None, None)
    monkeypatch.setattr("sys.argv", ["bench.py", "--power", "8", "--power-md", "p.md"])
    rows = [{"power": "forward", "calls": 5920, "seconds": 6.01, "samples": 9, "socket_power_w": 1339.0,
             "gfx_clock_mhz": 1799.0},
            {"power": "backward", "calls": 1840, "seconds": 6.0, "samples": 0, "socket_power_w": None,
             "gfx_clock_mhz": None}]
    line = {"config": {"workload": "long: B=1"}, "value": 900.0, "fwd_pct_peak": 43.0, "bwd_pct_peak": 34.0}
    p = tmp_path / "p.md"
    bench.write_power_md(str(p), rows, line)
    text = p.read_text()
    assert "python bench.py --power 8 --power-md p.md" in text
    assert "| forward | 5920 | 6.01 | 9 | 1339 | 1799 |" in text and "| backward | 1840 | 6.00 | 0 | - | - |" in text


def test_every_committed_summary_names_the_command_that_made_it():
    """Each profiles/*.md holds the bench.py (and for traces and counters the
    rocprofv3) command line that regenerates it, and names no file outside
    the repository's committed tree."""
    names = sorted(f for f in os.listdir(bench.PROFILES) if f.endswith(".md"))
    assert names
    for f in names:
        text = open(os.path.join(bench.PROFILES, f)).read()
        assert "python bench.py" in text, f
        if f.endswith(("_kernel_trace.md", "_counters.md")):
            assert "rocprofv3 " in text, f
        assert "_work/" not in text and "/root/reference" not in text, f
    t = json.load(open(bench.TRAFFIC_FILE))
    for wl, kernels in t["workloads"].items():
        for k, e in kernels.items():
            assert e["counters"] in names, (wl, k)
