"""bench.py's rocprofv3 summarisers on small synthetic CSVs (no GPU): the
copy calibration, the per-call traffic of a segmented prefill, the MFMA-busy
ratio, and the trace's phase and call split."""
import csv
import io
import os
import sys
from contextlib import redirect_stdout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for i, (name, grid, counter, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Agent_Id": "Agent 1", "Queue_Id": 1,
                        "Process_Id": 1, "Thread_Id": 1, "Grid_Size": grid, "Kernel_Id": 1,
                        "Kernel_Name": name, "Workgroup_Size": 256, "LDS_Block_Size": 0,
                        "Scratch_Size": 0, "VGPR_Count": 8, "Accum_VGPR_Count": 0, "SGPR_Count": 8,
                        "Counter_Name": counter, "Counter_Value": value, "Start_Timestamp": 0,
                        "End_Timestamp": 1})


def test_counter_summary(tmp_path):
    gib_kib = float(1 << 20)  # 1 GiB in KiB
    rows = [("__amd_rocclr_copyBuffer", 512, "FETCH_SIZE", 1.0)]            # small blit: ignored
    rows += [("__amd_rocclr_copyBuffer", 131072, "FETCH_SIZE", 0.5 * gib_kib)] * 3
    rows += [("__amd_rocclr_copyBuffer", 131072, "WRITE_SIZE", 1.0 * gib_kib)] * 3
    # 3 calls x 2 segments: each prep dispatch reads 100 MiB (counted at half) and writes 50 MiB
    rows += [("void kda::chunk_prep_kernel<...>(...)", 1, "FETCH_SIZE", 50 * 1024.0)] * 6
    rows += [("void kda::chunk_prep_kernel<...>(...)", 1, "WRITE_SIZE", 50 * 1024.0)] * 6
    rows += [("void kda::state_pass_kernel<...>(...)", 1, "FETCH_SIZE", 25 * 1024.0)] * 6
    rows += [("void kda::state_pass_kernel<...>(...)", 1, "WRITE_SIZE", 10 * 1024.0)] * 6
    for name, busy, gui in [("mfma32_loop(int, float*)", 800.0, 100.0),
                            ("void kda::chunk_prep_kernel<...>(...)", 40.0, 100.0),
                            ("void kda::state_pass_kernel<...>(...)", 120.0, 100.0)]:
        rows += [(name, 1, "SQ_VALU_MFMA_BUSY_CYCLES", busy), (name, 1, "GRBM_GUI_ACTIVE", gui)]
    # one counter file per pass, as rocprofv3 writes them
    _write_counters(str(tmp_path / "a"), [r for r in rows if r[2] == "FETCH_SIZE"])
    _write_counters(str(tmp_path / "b"), [r for r in rows if r[2] == "WRITE_SIZE"])
    _write_counters(str(tmp_path / "c"), [r for r in rows if r[2] not in ("FETCH_SIZE", "WRITE_SIZE")])
    buf = io.StringIO()
    with redirect_stdout(buf):
        out = bench.summarize([str(tmp_path)])
    text = buf.getvalue()
    assert "FETCH_SIZE reads 0.500 x" in text and "WRITE_SIZE 1.000 x" in text
    mib = float(1 << 20)
    pre = out["prefill"]
    # per call: 2 segments x (100 MiB + 50 MiB) read, 2 x (50 MiB + 10 MiB) written
    assert abs(pre["hbm_read_bytes_per_launch"] - 2 * 150 * mib) < 1.0
    assert abs(pre["hbm_write_bytes_per_launch"] - 2 * 60 * mib) < 1.0
    assert abs(pre["mfma_busy_rel_chunk_prep_kernel"] - 0.05) < 1e-12
    assert abs(pre["mfma_busy_rel_state_pass_kernel"] - 0.15) < 1e-12
    assert abs(pre["mfma_busy_rel_call"] - 0.1) < 1e-12


def test_trace_summary(tmp_path):
    path = tmp_path / "trace.csv"
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
              "Workgroup_Size_X", "LDS_Block_Size", "VGPR_Count", "Accum_VGPR_Count",
              "Scratch_Size"]
    rows, t = [], 0

    def k(name, dur, gap=1000):
        nonlocal t
        t += gap
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur,
                     "Grid_Size_X": 64, "Grid_Size_Y": 1, "Workgroup_Size_X": 256,
                     "LDS_Block_Size": 0, "VGPR_Count": 8, "Accum_VGPR_Count": 0, "Scratch_Size": 0})
        t += dur
    pause = 100_000_000  # 100 ms of host work between phases
    for c in range(2):    # headline prefill: 2 calls of 4 segments
        for s in range(4):
            k("chunk_prep_kernel", 90_000)
            k("state_pass_kernel", 100_000)
    k("mfma16_loop", 1_000_000, pause)
    k("mfma32_loop", 500_000)
    for _ in range(3):
        k("decode_kernel", 80_000, pause if _ == 0 else 1000)
    for s in range(8):   # long context: 1 call of 8 segments
        k("chunk_prep_kernel", 90_000, pause if s == 0 else 1000)
        k("state_pass_kernel", 300_000)
    k("chunk_prep_kernel", 20_000, pause)   # small prefill: 1 segment
    k("state_pass_kernel", 30_000)
    for s in range(4):   # per-head gate: 1 call
        k("chunk_prep_kernel", 91_000, pause if s == 0 else 1000)
        k("state_pass_kernel", 101_000)
    k("attnres_kernel", 390_000)            # no pause: split off by kernel kind
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fields)
        w.writeheader()
        w.writerows(rows)
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.summarize_trace(str(path))
    text = buf.getvalue()
    assert "| prefill_b4_h16_t16k | `chunk_prep_kernel` | 64 | 256 | 0 | 8/0 | 0 | 8 | 90.00 |" in text
    assert "| prefill_h16_t128k | `state_pass_kernel` | 64 | 256 | 0 | 8/0 | 0 | 8 | 300.00 |" in text
    assert "| attnres_l64_n4096_d4096 | `attnres_kernel` | 64 | 256 | 0 | 8/0 | 0 | 1 | 390.00 |" in text
    # whole calls: 4 x (90 + 1 + 100) + 3 gaps of 1 us = 767 us
    assert "| prefill_b4_h16_t16k | 2 | 767.0 |" in text
    assert "| prefill_h16_t128k | 1 |" in text
    assert "| prefill_b4_h16_t16k (per-head gate) | 1 |" in text


def test_lds_probe_cases_stay_in_bounds():
    """Every LDS probe case is accepted by kda_calibrate_lds: offsets below
    65216 bytes, aligned to the access width, two active lanes per pair case."""
    width = [4, 8, 16, 8, 4, 4, 8, 16, 4]
    cases = bench._lds_cases()
    assert len(cases) == 9 * 63 + 3 * 63 + 9 + 4
    for key, form, off in cases:
        assert len(off) == 64
        act = [o for o in off if o >= 0]
        assert all(o < 65216 and o % width[form] == 0 for o in act), key
        if key[0] in ("pair", "span"):
            assert len(act) == 2, key
        else:
            assert len(act) == 64, key


def test_lds_probe_summary(tmp_path):
    """The LDS model table from probe dispatches: a toy ground truth (lanes
    served together in groups of 16 for odd forms and 32 for even forms;
    32 banks for forms 0-4, 64 for 5-8) comes back out of the summary."""
    cases = bench._lds_cases()
    per_access = bench._LDS_BLOCKS * bench._LDS_ITERS
    rows = []
    for key, form, off in cases:
        if key[0] == "pair":
            _, f, j0, k = key
            grp = 16 if f % 2 else 32
            v = 1.0 if j0 // grp == k // grp else 0.0
        elif key[0] == "span":
            v = 1.0 if key[1] < 5 else 0.0
        else:
            v = 3.0
        rows.append((f"void (anonymous namespace)::lds_probe<{form}>(...)", 16, "SQ_LDS_BANK_CONFLICT",
                     v * per_access))
    _write_counters(str(tmp_path / "sq"), rows)
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench._summarize_lds([str(tmp_path / "sq")])
    text = buf.getvalue()
    assert "ds_read_b32     | j0=0: 0-31" in text
    assert "ds_read_b64     | j0=0: 0-15" in text
    assert "ds_read_b128    | j0=0: 0-31; j0=4: 0-31; j0=32: 32-63; j0=36: 32-63" in text
    lines = {ln.split("|")[0].strip("# ").strip(): ln.split("|")[2].strip() for ln in text.splitlines() if "|" in ln}
    assert lines["ds_read_b32"] == "32" and lines["ds_write_b32"] == "64"
    assert text.count(": 3.00") == 4
