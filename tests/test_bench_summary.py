"""The rocprofv3 summariser of bench.py (CPU only): byte calibration against the plain copy and the
matrix-core busy normalisation, on hand-made counter files."""
import csv
import json
import os

import bench

TRACE_COLS = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "VGPR_Count", "Accum_VGPR_Count", "LDS_Block_Size",
              "Start_Timestamp", "End_Timestamp"]
PMC_COLS = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
CHUNK = "void lz::(anonymous namespace)::chunk_kernel<lz::bf16_t, 128, false, false>(lz::BwdArgs, lz::bf16_t const*, float const*)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summary_scales_bytes_and_normalises_mfma(tmp_path):
    d = str(tmp_path / "prof")
    # a 1 ms chunk kernel at 2.4 GHz: 2.4e6 cycles on each of the 8 XCDs
    _write(f"{d}/kt/run_kernel_trace.csv", TRACE_COLS,
           [{"Kernel_Name": CHUNK, "Grid_Size_X": 8388608, "Workgroup_Size_X": 512, "VGPR_Count": 112,
             "Accum_VGPR_Count": 0, "LDS_Block_Size": 0, "Start_Timestamp": 0, "End_Timestamp": 1_000_000}])
    # the copy reads half its bytes in FETCH_SIZE units and all of them in WRITE_SIZE units
    _write(f"{d}/fetch/run_counter_collection.csv", PMC_COLS,
           [{"Kernel_Name": COPY, "Grid_Size": 131072, "Counter_Name": "FETCH_SIZE", "Counter_Value": 524288.0},
            {"Kernel_Name": CHUNK, "Grid_Size": 8388608, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000.0}])
    _write(f"{d}/write/run_counter_collection.csv", PMC_COLS,
           [{"Kernel_Name": COPY, "Grid_Size": 131072, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1048576.0},
            {"Kernel_Name": CHUNK, "Grid_Size": 8388608, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500.0}])
    insts = 1.0e6
    vals = {"SQ_VALU_MFMA_BUSY_CYCLES": 16 * insts, "SQ_INSTS_MFMA": insts, "GRBM_GUI_ACTIVE": 8 * 2.4e6,
            "SQ_INSTS_LDS": 2.0e6, "SQ_LDS_BANK_CONFLICT": 3.0e6, "SQ_BUSY_CYCLES": 1.0}
    _write(f"{d}/mfma/run_counter_collection.csv", PMC_COLS,
           [{"Kernel_Name": CHUNK, "Grid_Size": 8388608, "Counter_Name": k, "Counter_Value": v} for k, v in vals.items()])
    out = str(tmp_path / "out")
    bench.summarize_profiles(d, out)
    tr = json.load(open(f"{out}/traffic.json"))
    assert tr["_calibration"]["fetch_factor"] == 2.0 and tr["_calibration"]["write_factor"] == 1.0
    assert tr["chunk_kernel"]["read_bytes"] == 1000 * 1024 * 2 and tr["chunk_kernel"]["write_bytes"] == 500 * 1024
    c = json.load(open(f"{out}/counters.json"))["chunk_kernel"]
    # 16e6 busy SIMD-cycles over 2.4e6 cycles x 1024 SIMDs
    assert abs(c["mfma_busy_frac"] - 16e6 / (2.4e6 * 1024)) < 1e-4
    assert c["lds_bank_conflict_cycles_per_lds_inst"] == 1.5
    txt = open(f"{out}/train_8k_and_decode_counters.txt").read()
    assert "rocprofv3 --pmc FETCH_SIZE" in txt and "2.40" in txt   # the clock check: 2.4e6 cycles in 1 ms
    kt = open(f"{out}/train_8k_and_decode_kernel_trace.txt").read()
    assert "chunk_kernel<bf16_t, 128, false, false>" in kt and "16384" in kt and "1000.0" in kt


def test_all_sections_trace_groups_by_grid_and_drops_torch_kernels(tmp_path):
    d = str(tmp_path / "prof")
    row = lambda name, grid, t0, t1: {"Kernel_Name": name, "Grid_Size_X": grid, "Workgroup_Size_X": 256,
                                      "VGPR_Count": 64, "Accum_VGPR_Count": 0, "LDS_Block_Size": 0,
                                      "Start_Timestamp": t0, "End_Timestamp": t1}
    out_k = "void lz::(anonymous namespace)::out_kernel<lz::bf16_t, 128, false, false, false>(lz::FwdArgs)"
    torch_k = "void at::native::(anonymous namespace)::elementwise_kernel_with_index<int, at::native::arange>(int)"
    _write(f"{d}/kt/run_kernel_trace.csv", TRACE_COLS,
           [row(out_k, 16384 * 256, 0, 600_000), row(out_k, 16384 * 256, 0, 700_000),
            row(out_k, 4096 * 256, 0, 150_000), row(torch_k, 256, 0, 4_000)])
    with open(f"{d}/bench.log", "w") as f:
        f.write("noise\n" + json.dumps({"ms_per_step": 3.2, "value": 1.0e7, "kernels_ms": {"forward": 0.9},
                                        "decode": {"us_per_step": 65.0, "graph": {"us_per_step": 64.0}}}) + "\n")
    out = str(tmp_path / "out")
    bench.summarize_trace(d, out, f"{d}/bench.log")
    txt = open(f"{out}/bench_all_sections_kernel_trace.txt").read()
    rows = [l for l in txt.splitlines() if l.startswith("out_kernel")]
    # one row per grid, the two 16384-workgroup launches averaged (650 us), the torch kernel left out
    assert len(rows) == 2 and "650.0" in rows[0] and "16384" in rows[0] and "4096" in rows[1]
    assert "at::" not in txt.split("\n\n")[1]
    assert "decode: us_per_step 65.0, graph.us_per_step 64.0" in txt
