"""The profile summaries' host logic on synthetic rocprofv3 CSV rows: the
per-dispatch sums and means, the copy-scaled traffic, the derived counter
rates, and the source hash the bench checks before it reuses a traffic
figure."""
import csv
import os

import pytest

from vocab_wide_logit_amd import profiling as P

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_per_dispatch_sums_instances_and_averages_dispatches(tmp_path):
    p = str(tmp_path / "c.csv")
    _write(p, [(1, "void vwl::k<2>(P)", 1024, 256, "X", 3.0), (1, "void vwl::k<2>(P)", 1024, 256, "X", 5.0),
               (2, "void vwl::k<2>(P)", 1024, 256, "X", 4.0), (3, "void vwl::other(P)", 256, 256, "X", 100.0),
               (4, "void vwl::k<2>(P)", 512, 256, "X", 50.0)])
    mean, n = P._per_dispatch(p, "X", r"k<2>", grid_wgs=4)
    assert (mean, n) == (6.0, 2)  # (3 + 5) and 4 over the two 4-workgroup dispatches
    mean, n = P._per_dispatch(p, "X", r"k<2>")
    assert n == 3 and mean == pytest.approx((8.0 + 4.0 + 50.0) / 3)
    with pytest.raises(ValueError):
        P._per_dispatch(p, "Y", r"k<2>")


def test_counter_summary_rates(tmp_path):
    p = str(tmp_path / "c.csv")
    rows = []
    for d in (1, 2):
        rows += [(d, "void vwl::lmhead_jsd_kernel(P)", 1024, 256, "TCC_HIT_sum", 80.0),
                 (d, "void vwl::lmhead_jsd_kernel(P)", 1024, 256, "TCC_MISS_sum", 20.0),
                 (d, "void vwl::lmhead_jsd_kernel(P)", 1024, 256, "GRBM_GUI_ACTIVE", 8000.0),
                 (d, "void vwl::lmhead_jsd_kernel(P)", 1024, 256, "TA_BUSY_avr", 250.0),
                 (d, "void vwl::lmhead_jsd_kernel(P)", 1024, 256, "SQ_VALU_MFMA_BUSY_CYCLES", 1024.0 * 500.0)]
    _write(p, rows)
    out = str(tmp_path / "s.txt")
    r = P.summarize_counters(p, out, "cmd", r"lmhead_jsd_kernel", "w")
    assert r["dispatches"] == 2
    assert r["l2_hit_fraction"] == pytest.approx(0.8)
    assert r["ta_busy"] == pytest.approx(0.25)   # 250 busy of 8000 / 8 cycles per die
    assert r["mfma_busy"] == pytest.approx(0.5)  # 500 cycles per SIMD of 1000
    text = open(out).read()
    assert "command: cmd" in text and "l2_hit_fraction" in text


def test_traffic_scaled_by_the_copy(tmp_path):
    f, w = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    kib = 1024.0
    copy = P.COPY_BYTES
    # the counters read half the copy's bytes for FETCH and all of them for WRITE
    _write(f, [(1, "void at::neg_kernel(x)", 4096, 256, "FETCH_SIZE", 0.5 * copy / kib),
               (2, "void vwl::asym_rows_kernel<1, 4, 0, 0>(P)", 760 * 256, 256, "FETCH_SIZE", 0.5 * 1000.0 / kib)])
    _write(w, [(1, "void at::neg_kernel(x)", 4096, 256, "WRITE_SIZE", copy / kib),
               (2, "void vwl::asym_rows_kernel<1, 4, 0, 0>(P)", 760 * 256, 256, "WRITE_SIZE", 10.0 / kib)])
    r = P.summarize_pmc(f, w, str(tmp_path / "t.txt"), "cmd", "asym", grid_wgs=760)
    assert r["fetch_bytes_per_launch"] == pytest.approx(1000.0)
    assert r["write_bytes_per_launch"] == pytest.approx(10.0)
    # the bench reuses the figure only while the kernel sources match
    assert P.read_traffic(str(tmp_path / "t.txt"), "asym") == pytest.approx(1010.0)


def test_source_hash_tracks_the_kernel_sources():
    h = P.source_hash("asym")
    assert len(h) == 16 and h == P.source_hash("asym")
    assert h != P.source_hash("rapid")
