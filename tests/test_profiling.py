"""CPU checks of the rocprofv3 summary helpers (profiling.py): the kernel
source hash ignores comments and spacing but not code, counter rows are
summed per dispatch, and traffic() scales each kernel's counted bytes by the
calibration copy's known size."""
import csv
import os

import pytest

from combine_routing_histogram_amd import profiling as prof


def test_hash_ignores_comments_and_spacing_only():
    base = "int f(int x) {\n  return x + 1; // one\n}\n/* block */\n"
    assert prof.kernel_source_hash(base) == prof.kernel_source_hash(
        "int f(int x)   {  return x + 1;\n\n} // other words\n")
    assert prof.kernel_source_hash(base) != prof.kernel_source_hash(base.replace("+ 1", "+ 2"))


def _write_counters(d, counter, rows):
    """rows: (kernel, dispatch id, value) -> a rocprofv3-style counter csv."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "c_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for k, i, v in rows:
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": counter,
                        "Counter_Value": v})
            # a row of another counter in the same file is ignored
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": "OTHER",
                        "Counter_Value": 1e9})


def test_read_counters_sums_dimensions_per_dispatch(tmp_path):
    d = str(tmp_path / "f")
    _write_counters(d, "FETCH_SIZE", [("k_a", 1, 10.0), ("k_a", 1, 5.0), ("k_a", 2, 7.0),
                                      ("k_b", 3, 2.0)])
    got = prof.read_counters(d, "FETCH_SIZE")
    assert sorted(got["k_a"]) == [7.0, 15.0] and got["k_b"] == [2.0]
    with pytest.raises(FileNotFoundError):
        prof.read_counters(str(tmp_path / "missing"), "FETCH_SIZE")


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    fd, wd = str(tmp_path / "f"), str(tmp_path / "w")
    calib = 512 << 20
    # the copy kernel: a small upload, then the calibration copy, which the
    # counters see as 2x its bytes read and exactly its bytes written (KiB)
    _write_counters(fd, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1, 4.0),
                                       ("__amd_rocclr_copyBuffer", 2, 2 * calib / 1024),
                                       ("void epdc::k_combine<8, 2, 0>", 3, 1000.0),
                                       ("void epdc::k_combine<8, 2, 0>", 4, 1200.0),
                                       ("void epdc::k_combine<8, 2, 0>", 5, 1100.0)])
    _write_counters(wd, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1, 4.0),
                                       ("__amd_rocclr_copyBuffer", 2, calib / 1024),
                                       ("void epdc::k_combine<8, 2, 0>", 3, 300.0),
                                       ("void epdc::k_combine<8, 2, 0>", 4, 300.0),
                                       ("void epdc::k_combine<8, 2, 0>", 5, 300.0)])
    t = prof.traffic(fd, wd, "k_combine", calib)
    assert t["fetch_scale"] == pytest.approx(0.5) and t["write_scale"] == pytest.approx(1.0)
    # median fetch 1100 KiB at half scale + 300 KiB written
    assert t["hbm_bytes_per_launch"] == pytest.approx(1100 * 1024 * 0.5 + 300 * 1024)
    assert t["launches_matched"] == ["void epdc::k_combine<8, 2, 0>"]
    assert t["kernel_source_sha256_16"] == prof.kernel_source_hash()
    with pytest.raises(KeyError):
        prof.traffic(fd, wd, "k_not_there", calib)
