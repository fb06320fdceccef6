"""CPU tests of the profile summarisers that turn rocprofv3 output into the
committed summaries: each runs on a small database or table built here with
known contents, so the figures they print can be checked by hand."""
import sqlite3

from long_context_lm_chunk_amd import profile_summary as PS
from long_context_lm_chunk_amd import traffic_summary as TS


def _trace_db(path, rows):
    c = sqlite3.connect(path)
    c.execute("create table kernels (stream_id int, start int, end int, name text, duration int)")
    c.executemany("insert into kernels values (?, ?, ?, ?, ?)", [(s, a, b, n, b - a) for s, a, b, n in rows])
    c.commit()
    c.close()


def test_kernel_table_totals_and_shares(tmp_path):
    db = str(tmp_path / "k.db")
    # times in ns: kernel A 3 x 3 us, kernel B 1 x 6 us
    _trace_db(db, [(0, 0, 3000, "A"), (0, 4000, 7000, "A"), (1, 0, 6000, "B"), (0, 8000, 11000, "A")])
    out = PS.summarise(db, per=2)
    assert "Total kernel time 0.0 ms over 4 dispatches" in out
    lines = [ln for ln in out.splitlines() if ln.startswith("| `")]
    assert lines[0].startswith("| `A` | 3 | 0.01 | 1.5 |")
    assert lines[0].endswith("| 3.0 | 60.0% |")      # avg 3 us, 9 of 15 us
    assert lines[1].startswith("| `B` | 1 |") and lines[1].endswith("| 6.0 | 40.0% |")


def test_stream_occupancy_window_and_gaps(tmp_path):
    db = str(tmp_path / "s.db")
    ms = 1_000_000
    rows = [
        (0, 0, 1 * ms, "embed_k"),            # first unit (before the window)
        (0, 10 * ms, 12 * ms, "embed_k"),     # window starts here (index 1)
        (0, 12 * ms + 5000, 14 * ms, "gemm"),   # 5 us gap
        (0, 16 * ms, 20 * ms, "gemm"),        # 2 ms gap
        (1, 11 * ms, 13 * ms, "attn"),
        (1, 12 * ms, 15 * ms, "attn"),        # overlaps the previous one on its stream
        (0, 30 * ms, 31 * ms, "dgemv"),       # stop marker: not in the window
    ]
    _trace_db(db, rows)
    out = PS.streams(db, "embed_k", 1, "dgemv")
    assert "Window: 10.0 ms" in out
    r0 = next(ln for ln in out.splitlines() if ln.startswith("| 0 |"))
    r1 = next(ln for ln in out.splitlines() if ln.startswith("| 1 |"))
    # stream 0: busy 2 + 1.995 + 4 ms of the 10 ms window; one gap over 1 ms (2 ms), one below (5 us)
    f0 = [x.strip() for x in r0.strip("|").split("|")]
    assert f0[1] == "3" and f0[2] == "8.0" and f0[3] == "80.0%" and f0[5] == "1" and f0[6] == "2.0"
    assert f0[7] == "0.0"                            # the 5 us gap, in ms
    # stream 1: the union of two overlapping dispatches, 11..15 ms
    f1 = [x.strip() for x in r1.strip("|").split("|")]
    assert f1[1] == "2" and f1[2] == "4.0" and f1[4] == "100.0%" and f1[5] == "0"


def test_traffic_scaled_by_the_copy_probe(tmp_path):
    mib = 4
    f, w = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    for path, counter, probe_kib, kern_kib in ((f, "FETCH_SIZE", mib * 1024 / 2, 300.0),
                                                (w, "WRITE_SIZE", mib * 1024, 100.0)):
        c = sqlite3.connect(path)
        c.execute("create table counters_collection (dispatch_id int, kernel_name text, grid_size int, "
                  "counter_name text, value real)")
        c.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", [
            (0, "at::native::MulFunctor copy", 1 << 20, counter, probe_kib),
            (1, "gemm256_kernelILi4EDF16b", 256, counter, kern_kib),
            (2, "gemm256_kernelILi4EDF16b", 256, counter, kern_kib),
            (3, "other_kernel", 64, counter, 1e6),
        ])
        c.commit()
        c.close()
    out = TS.summarise(f, w, "gemm256_kernelILi4EDF16b", probe_mib=mib, shapes=[("t", 16, 16, 8)],
                       bytes_per_weight=10.0)
    assert "factor 0.500" in out and "factor 1.000" in out
    # FETCH counts half the bytes: 300 KiB read as 600 KiB; WRITE 100 KiB as is
    assert "| t | 2 | 0.6 MB | 0.1 MB | 0.7 MB |" in out
    # algorithmic: 10 B x 16 x 16 + 2 B x (16 + 16) x 8 = 3072 B
    assert "0.0 MB |" in out


def test_counter_table_formulas(tmp_path):
    from long_context_lm_chunk_amd import pmc_summary as PM
    path = str(tmp_path / "m_counter_collection.csv")
    # one dispatch of 1 us; 8 XCDs report 1000 active cycles each; half of
    # the 1024 SIMDs' cycles MFMA-busy, a quarter of the 256 CUs' VALU busy;
    # 1e6 bf16 MFMA MOPs (512 flops each) in 1 us = 512 TFLOP/s
    counters = {"GRBM_GUI_ACTIVE": 8000, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1000 * 1024,
                "SQ_ACTIVE_INST_VALU": 0.25 * 256 * 1000, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1e6}
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
        for k, v in counters.items():
            f.write(f"7,probe_kernel(int),{k},{v},1000,2000\n")
    out = PM.summarise([path])
    row = next(ln for ln in out.splitlines() if ln.startswith("| `probe_kernel`"))
    assert row == "| `probe_kernel` | 1 | 0.00 | 1.0 | 100.0% | 50.0 | 25.0 | 512 |"
