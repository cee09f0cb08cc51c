"""Host logic of the measurement helpers (no GPU): the kernel-trace summary of
boundary dispatches beside decode launches."""
import csv
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from linear_attention_recurrent_gdn_amd import profiling  # noqa: E402

DEC = "void lq::decode_q8_kernel<128, false, 6, 2, 0, false, true>(lq::DecodeArgs)"
FLUSH = "void lq::materialize_kernel<128, false, 1, false>(lq::MatArgs)"
INIT = "void lq::materialize_kernel<128, false, 0, false>(lq::MatArgs)"


def _trace(path, rows):
    keys = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=keys)
        w.writeheader()
        for name, s, e, grid in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": s, "End_Timestamp": e,
                        "Workgroup_Size_X": 512, "Grid_Size_X": grid * 512})


def test_overlap_summary_classifies_dispatches(tmp_path):
    # times in ns: decodes back to back; one boundary (96 workgroups) spans the
    # second and third decode, one alone (256) after all of them; an init
    # dispatch is not a boundary
    rows = [(INIT, 0, 500, 256), (DEC, 1000, 2000, 8192), (DEC, 2000, 4000, 8192), (DEC, 4000, 6000, 8192),
            (DEC, 6000, 7000, 8192), (FLUSH, 2500, 5000, 96), (FLUSH, 9000, 9800, 256)]
    tr = tmp_path / "kt.csv"
    _trace(tr, rows)
    text = profiling.overlap(str(tr), "cmd", str(tmp_path / "out.txt"))
    assert "beside decode launches: 1, grid [96] workgroups, mean 2.5 us" in text
    assert "boundary dispatches alone: 1, grid [256] workgroups, mean 0.8 us" in text
    # span of the overlapped boundary: decodes starting in [2500, 5000): only the third
    assert "decode launches in that span: 1; beside a boundary 1, mean 2.00 us; alone 0" in text
