"""Host tests of the profile-summary tool (matmul_affine_qmv_amd/traffic.py):
the step timeline of a kernel trace, on small hand-written CSV files."""
import csv

from matmul_affine_qmv_amd import traffic

FIELDS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]


def _trace(path, events):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, b, e in events:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": b, "End_Timestamp": e})


def test_timeline_durations_and_gaps(tmp_path):
    # two steps of kernels A (2 us) then B (3 us), 1 us apart inside a step and
    # 5 us between steps; a foreign kernel and an earlier warm-up step are ignored
    ev = [("void qmx::A(int)", 0, 2000), ("void qmx::B(int)", 2000, 5000),          # warm-up step
          ("void qmx::A(int)", 10000, 12000), ("other", 12000, 12500), ("void qmx::B(int)", 13000, 16000),
          ("void qmx::A(int)", 21000, 23000), ("void qmx::B(int)", 24000, 27000)]
    p = tmp_path / "run_kernel_trace.csv"
    _trace(p, ev)
    md = traffic.timeline_markdown(str(p), per_step=2, steps=2)
    rows = [l for l in md.splitlines() if l.startswith("| 0 ") or l.startswith("| 1 ")]
    assert rows[0] == "| 0 | `qmx::A` | 2.00 | 5.00 |"     # gap from the previous step's B
    assert rows[1] == "| 1 | `qmx::B` | 3.00 | 1.00 |"
    assert "Step span (first kernel's start to last kernel's end, median): 6.0 µs" in md
    assert "sum of its kernels' durations: 5.0 µs" in md


def test_timeline_needs_enough_kernels(tmp_path):
    p = tmp_path / "run_kernel_trace.csv"
    _trace(p, [("void qmx::A(int)", 0, 10)])
    try:
        traffic.timeline_markdown(str(p), per_step=2, steps=1)
    except SystemExit as e:
        assert "fewer than 2" in str(e)
    else:
        raise AssertionError("expected SystemExit")
