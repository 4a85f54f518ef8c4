"""Host-side checks of the rocprofv3 summaries (no GPU): the per-kernel
counter averages and derived figures, the traffic summary's round trip, and
the committed traffic summary that bench.py reads."""
import csv
import os

import pytest

from linear_cross_entropy_cce_amd import profiling as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_agent_info.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Num_Xcc", "Simd_Count"])
        w.writeheader()
        w.writerow({"Name": "gfx950", "Num_Xcc": 8, "Simd_Count": 1024})
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _dispatch(did, kernel, ns, counters):
    # rocprofv3 writes one row per counter (and per XCD instance; two halves here)
    out = []
    for name, value in counters.items():
        for half in (0.5, 0.5):
            out.append({"Dispatch_Id": did, "Kernel_Name": kernel, "Counter_Name": name,
                        "Counter_Value": value * half, "Start_Timestamp": 1000, "End_Timestamp": 1000 + ns})
    return out


def test_counters_two_kernels(tmp_path):
    d = str(tmp_path / "pmc")
    counters = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
    # kernel a: 2 dispatches of 1 ms at 1.5 GHz on 8 XCDs, MFMA busy half of 1024 SIMDs' cycles
    cyc = 1.5e6
    a = {"SQ_INSTS_MFMA": 1e6, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cyc * 1024, "GRBM_GUI_ACTIVE": 8 * cyc}
    b = {"SQ_INSTS_MFMA": 4e6, "SQ_VALU_MFMA_BUSY_CYCLES": 0.8 * 2 * cyc * 1024, "GRBM_GUI_ACTIVE": 8 * 2 * cyc}
    rows = _dispatch(1, "void k_a<int>(int)", 1_000_000, a) + _dispatch(2, "void k_a<int>(int)", 1_000_000, a)
    rows += _dispatch(3, "Cijk_gemm", 2_000_000, b) + _dispatch(9, "other_kernel", 5, a)
    _write_counters(d, rows)
    out = str(tmp_path / "c.md")
    res = P.write_counters_md(out, d, "cmd", "title", kernels=("k_a", "Cijk"), counters=counters)
    assert res["k_a"]["dispatches"] == 2 and res["Cijk"]["dispatches"] == 1
    assert res["k_a"]["clock_ghz"] == pytest.approx(1.5)
    assert res["Cijk"]["clock_ghz"] == pytest.approx(1.5)
    assert res["k_a"]["mfma_busy"] == pytest.approx(0.5)
    assert res["Cijk"]["mfma_busy"] == pytest.approx(0.8)
    assert res["k_a"]["cycles_per_mfma"] == pytest.approx(0.5 * cyc * 1024 / 1e6)
    text = open(out).read()
    assert "`void k_a<int>`" in text and "`Cijk_gemm`" in text and "other_kernel" not in text
    assert "50.0%" in text and "80.0%" in text


def test_counters_missing_kernel(tmp_path):
    d = str(tmp_path / "pmc")
    _write_counters(d, _dispatch(1, "k_a", 10, {"GRBM_GUI_ACTIVE": 8.0}))
    with pytest.raises(RuntimeError):
        P.write_counters_md(str(tmp_path / "c.md"), d, "cmd", "t", kernels=("k_a", "absent"),
                            counters=("GRBM_GUI_ACTIVE",))


def test_traffic_summary_round_trip(tmp_path):
    s = {"FETCH_SIZE": {"kernel_kib": 100.0, "copy_kib": 50.0, "factor": 2.0, "bytes": 204800.0},
         "WRITE_SIZE": {"kernel_kib": 10.0, "copy_kib": 50.0, "factor": 1.0, "bytes": 10240.0},
         "traffic_bytes": 215040.0}
    path = str(tmp_path / "t.md")
    P.write_md(path, s, 1024, "rocprofv3 --pmc COUNTER -- x")
    got = P.load(path)
    assert got == (215040.0, P.sources_hash())


def test_committed_traffic_summary_parses():
    got = P.load(os.path.join(ROOT, "profiles", "k_fwd4_gemma2_2b_head_traffic.md"))
    assert got is not None
    nbytes, h = got
    # at least the algorithmic bytes of one launch (H and E once, bf16)
    assert nbytes >= 2 * (8192 + 256000) * 2304
    assert len(h) == 16


def test_step_traffic_sums_dispatches(tmp_path):
    # two steps, a kernel dispatched three times a step, and a 1 MiB copy that
    # the counter reads as 512 KiB (factor 2)
    for counter, per in (("FETCH_SIZE", 100.0), ("WRITE_SIZE", 40.0)):
        d = str(tmp_path / counter)
        rows = []
        for i in range(6):
            rows += _dispatch(i, "void cce::k_grad_pass<unsigned short, true>(x)", 1000, {counter: per})
        rows += _dispatch(99, "__amd_rocclr_copyBuffer", 1000, {counter: 512.0})
        _write_counters(d, rows)
    s = P.step_traffic(str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"), 1 << 20, ["k_grad_pass"], 2)
    v = s["k_grad_pass"]
    assert v["FETCH_SIZE"]["dispatches"] == 6
    assert v["FETCH_SIZE"]["bytes_per_step"] == pytest.approx(3 * 100.0 * 1024 * 2)
    assert v["WRITE_SIZE"]["bytes_per_step"] == pytest.approx(3 * 40.0 * 1024 * 2)
    assert v["traffic_bytes_per_step"] == pytest.approx(3 * 140.0 * 1024 * 2)
    out = tmp_path / "t.md"
    P.write_step_traffic_md(str(out), s, 1 << 20, 2, "rocprofv3 --pmc COUNTER -- cmd", "title",
                            str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"))
    assert "k_grad_pass" in out.read_text()
