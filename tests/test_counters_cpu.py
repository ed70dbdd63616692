"""The counter summaries that back the profiles, checked on the CPU with
synthetic rocprofv3 output: phases split at the one-block marker copies,
per-kernel means, the matrix-core busy share and the byte scaling."""
import csv
import os

from ternary_weight_linear_quant_amd import counters as C

FIELDS = ["Process_Id", "Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
          "Counter_Value"]


def _write_pass(d, per_phase, counters_of):
    """One marker copy before every phase and after the last; `per_phase`
    maps a phase to its (kernel name, grid) dispatches."""
    os.makedirs(d, exist_ok=True)
    rows, did = [], 0

    def add(name, grid, vals):
        nonlocal did
        did += 1
        for c, v in vals.items():
            rows.append({"Process_Id": 1, "Dispatch_Id": did, "Kernel_Name": name,
                         "Grid_Size": grid, "Counter_Name": c, "Counter_Value": v})

    marker = ("bl::k_calib_copy(int const*, int*, long)", 64)
    for ph in C.PHASE_ORDER:
        add(*marker, {c: 0.0 for c in counters_of(None)})
        for name, grid in per_phase.get(ph, []):
            add(name, grid, counters_of(name))
    add(*marker, {c: 0.0 for c in counters_of(None)})
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        w.writerows(rows)


def test_busy_share_and_instruction_ratio(tmp_path):
    kern = "void bl::k_gemm<128, 512, 1, 8, 3, 2, false, 1>(signed char const*)"

    def vals(name):
        v = {c: 0.0 for c in C.BUSY_COUNTERS}
        if name == kern:
            # 1000 active cycles per XCD; each SIMD's matrix core busy 250.
            v.update({"GRBM_GUI_ACTIVE": 8000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 250.0 * 1024,
                      "SQ_INSTS_MFMA": 100.0, "SQ_INSTS_VALU": 450.0})
        return v

    d = str(tmp_path / "busy")
    _write_pass(d, {"gemm_prefill_4096": [(kern, 1024), (kern, 1024)]}, vals)
    out = C.busy(d, "CMD")
    row = [ln for ln in out.splitlines() if ln.startswith("| gemm_prefill_4096 |")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[1] == "k_gemm<128, 512, 1, 8, 3, 2, false, 1>"
    assert cells[2] == "2"           # dispatches
    assert cells[3] == "25.0%"       # 250 / 1000
    assert cells[4] == "4.50"        # VALU per MFMA
    assert "CMD" in out


def test_phases_require_every_marker(tmp_path):
    d = str(tmp_path / "short")
    os.makedirs(d)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        w.writerow({"Process_Id": 1, "Dispatch_Id": 1,
                    "Kernel_Name": "bl::k_calib_copy(int const*, int*, long)", "Grid_Size": 64,
                    "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 1})
    try:
        C.busy(d, "CMD")
    except SystemExit as e:
        assert "phases" in str(e)
    else:
        raise AssertionError("a pass with missing phases must be refused")
