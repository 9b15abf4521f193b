"""Host-side checks of the profile summariser's parsing (no GPU, no profiler):
kernel-trace statistics, counter values per dispatch, and kernel families."""
import csv

import pytest

from decode_attention_03_amd import rocprof_summary as rs


def _write(path, fields, rows):
    with open(path, "w", newline="", encoding="utf-8") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_trace_stats(tmp_path):
    p = tmp_path / "trace.csv"
    rows = [{"Kernel_Name": "split_valu_kernel<...>", "Start_Timestamp": 1000, "End_Timestamp": 11000},
            {"Kernel_Name": "split_valu_kernel<...>", "Start_Timestamp": 20000, "End_Timestamp": 26000},
            {"Kernel_Name": "combine_kernel<128>", "Start_Timestamp": 27000, "End_Timestamp": 31000}]
    _write(p, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    st = rs.trace_stats(str(p))
    assert [r["kernel"] for r in st] == ["split_valu_kernel<...>", "combine_kernel<128>"]
    split, comb = st
    assert split["calls"] == 2 and split["avg_us"] == pytest.approx(8.0)
    assert split["min_us"] == pytest.approx(6.0) and split["max_us"] == pytest.approx(10.0)
    assert comb["calls"] == 1 and comb["avg_us"] == pytest.approx(4.0)
    assert split["share"] == pytest.approx(16 / 20) and comb["share"] == pytest.approx(4 / 20)


def test_counter_per_dispatch_sums_instances_and_averages_dispatches(tmp_path):
    """A counter appears once per hardware instance of a dispatch: the value
    of a dispatch is their sum, and the result the mean over dispatches of
    the matching (else the most dispatched) kernel."""
    p = tmp_path / "pmc.csv"
    rows = []
    for d, vals in ((1, (10, 20)), (2, (30, 40)), (3, (5, 5))):
        for v in vals:
            rows.append({"Dispatch_Id": d, "Kernel_Name": "split" if d < 3 else "combine",
                         "Counter_Name": "FETCH_SIZE", "Counter_Value": v})
    rows.append({"Dispatch_Id": 1, "Kernel_Name": "split", "Counter_Name": "WRITE_SIZE",
                 "Counter_Value": 999})
    _write(p, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    mean, n, name = rs.counter_per_dispatch(str(p), "FETCH_SIZE")
    assert (mean, n, name) == (50.0, 2, "split")
    mean, n, name = rs.counter_per_dispatch(str(p), "FETCH_SIZE", lambda k: k == "combine")
    assert (mean, n, name) == (10.0, 1, "combine")
    with pytest.raises(RuntimeError):
        rs.counter_per_dispatch(str(p), "FETCH_SIZE", lambda k: k == "missing")


def test_kernel_families_and_json_line():
    assert rs.family_of("void fd::(anonymous namespace)::split_valu_kernel<2, 128>") == "split_valu"
    assert rs.family_of("void fd::(anonymous namespace)::split_mfma_tiled_kernel<2>") == "split_mfma"
    assert rs.family_of("void fd::(anonymous namespace)::combine_slots_kernel<64>") == "combine"
    assert rs.family_of("__amd_rocclr_copyBuffer") is None
    assert rs.last_json_line('noise\n{"a": 1}\nmore\n{"b": 2}\n') == {"b": 2}
