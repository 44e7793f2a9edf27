"""Host-side bookkeeping of the measurement tools (no GPU): the HBM traffic
records that bench.py reports per kernel and workload, and the algorithmic
work it divides by."""
import csv
import json
import types

from exact_io_aware_07_amd import profiling
from exact_io_aware_07_amd import workloads as W

DKDV = "void fa::(anonymous namespace)::dkdv_kernel<fa::BF16, 64, false>(fa::BwdArgs)"
FWD = "void fa::(anonymous namespace)::fwd_mfma_kernel<fa::BF16, 64, false, false, false>(fa::FwdArgs)"
COPY = "void at::native::elementwise_kernel_copy<128>(int)"


def _csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
    return str(path)


def _args(tmp_path, workload, fetch_kib, write_kib):
    copy_bytes = 1 << 20
    return types.SimpleNamespace(
        # the copy reads and writes 1 MiB; its counters read 512 KiB fetched
        # and 1024 KiB written, so fetched KiB count double and written once
        copy_fetch=_csv(tmp_path / "cf.csv", "FETCH_SIZE", [(COPY, 512.0)]),
        copy_write=_csv(tmp_path / "cw.csv", "WRITE_SIZE", [(COPY, 1024.0)]),
        fetch=_csv(tmp_path / f"f_{workload}.csv", "FETCH_SIZE",
                   [(DKDV, fetch_kib), (DKDV, fetch_kib + 2.0), (FWD, 10.0)]),
        write=_csv(tmp_path / f"w_{workload}.csv", "WRITE_SIZE", [(DKDV, write_kib), (FWD, 4.0)]),
        copy_bytes=copy_bytes, workload=workload, cmd="rocprofv3 ...",
        out_md=str(tmp_path / f"{workload}.md"), out_json=str(tmp_path / "traffic.json"))


def test_traffic_keeps_one_record_per_workload_scaled_by_the_copy(tmp_path):
    profiling.traffic(_args(tmp_path, "a", 100.0, 50.0))
    profiling.traffic(_args(tmp_path, "b", 200.0, 70.0))
    path = str(tmp_path / "traffic.json")
    assert sorted(json.load(open(path))["workloads"]) == ["a", "b"]
    # dkdv on workload a: mean of 100 and 102 KiB fetched (x 2), 50 KiB written (x 1)
    assert profiling.traffic_record(path, "a", "dkdv") == (101.0 * 1024 * 2, 50.0 * 1024)
    assert profiling.traffic_record(path, "b", "dkdv") == (201.0 * 1024 * 2, 70.0 * 1024)
    assert profiling.traffic_record(path, "b", "fwd") == (10.0 * 1024 * 2, 4.0 * 1024)
    assert profiling.traffic_record(path, "c", "dkdv") is None
    assert profiling.traffic_record(path, "a", "dq") is None


def test_traffic_record_is_dropped_once_the_kernel_source_changes(tmp_path):
    profiling.traffic(_args(tmp_path, "a", 100.0, 50.0))
    path = tmp_path / "traffic.json"
    rec = json.load(open(path))
    rec["workloads"]["a"]["kernels"]["dkdv"]["source_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert profiling.traffic_record(str(path), "a", "dkdv") is None
    assert profiling.traffic_record(str(path), "a", "fwd") is not None


def test_traffic_file_of_the_old_single_record_form_is_replaced(tmp_path):
    (tmp_path / "traffic.json").write_text(json.dumps({"workload": "x", "kernels": {}}))
    profiling.traffic(_args(tmp_path, "a", 100.0, 50.0))
    assert list(json.load(open(tmp_path / "traffic.json"))["workloads"]) == ["a"]


def test_kernel_work_of_the_three_kernels_is_the_algorithmic_step():
    # forward: two products of 2d FLOPs per visible pair; backward: five
    # more (the dQ kernel is credited with one, the dK/dV kernel with four)
    import bench
    for w in (W.GPT2, W.LONG_BWD, W.TRADE_BWD):
        step = sum(bench.kernel_work(k, w) for k in ("fwd", "dq", "dkdv"))
        assert step == 3.5 * bench.fwd_flops(w)
        assert bench.kernel_work("dkdv", w) == 2.0 * bench.fwd_flops(w)
