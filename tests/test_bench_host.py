"""Host logic of bench.py (CPU): the one-GPU contract and the HBM-traffic records that
turn rocprofv3 --pmc counter files into profiles/traffic.json."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

HALO = "_ZN3c2d14halo3x3_kernelIDF16bLi64ELi4ELi2ELi2ELi8ELb0EEEvNS_8ConvArgsEiiiNS_8HaloPoolE"
GEMM = "_ZN3c2d17igemm_nhwc_kernelIDF16bLi64ELi64ELi2ELi2ELi3ELi1ELb1ELb0ELb0EEEvNS_8ConvArgsEiiPf"
COPY = "__amd_rocclr_copyBuffer"


def _counters(path, counter, launches):
    """A counter_collection.csv as rocprofv3 writes it: one row per dispatch and counter
    instance; `launches` is [(kernel, dispatches, KiB per dispatch)]."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        d = 0
        for kernel, n, kib in launches:
            for _ in range(n):
                d += 1
                # two instances per dispatch (e.g. two XCDs), summed by the reader
                w.writerow([d, kernel, counter, kib / 2])
                w.writerow([d, kernel, counter, kib / 2])


@pytest.fixture
def tree(tmp_path, monkeypatch):
    """bench.ROOT pointed at a scratch tree that shares the library's sources (for the
    source hashes) but has its own profiles/."""
    os.symlink(os.path.join(ROOT, "conv2d_bias_activation_amd"), tmp_path / "conv2d_bias_activation_amd")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = tmp_path / "pmc"
    # a 256 MiB copy whose FETCH_SIZE reads half the bytes (scale 2) and WRITE_SIZE all (scale 1)
    _counters(src / "copy_fetch", "FETCH_SIZE", [(COPY, 10, 131072.0)])
    _counters(src / "copy_write", "WRITE_SIZE", [(COPY, 10, 262144.0)])
    # the kernel run also launches copies (weights to the device), more often than the kernel
    _counters(src / "fetch", "FETCH_SIZE", [(COPY, 30, 4.0), (HALO, 20, 1000.0), (GEMM, 2, 77.0)])
    _counters(src / "write", "WRITE_SIZE", [(COPY, 30, 4.0), (HALO, 20, 500.0), (GEMM, 2, 55.0)])
    return tmp_path, src


def test_traffic_record_picks_the_plans_kernel_and_scales_by_the_copy(tree):
    root, src = tree
    bench.write_traffic(str(src), 256, "halo3x3_nhwc bf16 th4 co64 w8")
    rec = json.load(open(root / "profiles" / "traffic.json"))
    assert rec["copy"]["fetch_scale"] == 2.0 and rec["copy"]["write_scale"] == 1.0
    k = rec["kernels"]["halo3x3_nhwc bf16 th4 co64 w8"]
    assert k["kernel"] == HALO  # not the copy kernel, which launched more often
    assert k["fetch_kib"] == 1000.0 and k["write_kib"] == 500.0
    assert k["bytes_per_launch"] == (1000 * 2 + 500) * 1024
    # a tuned choice of the same plan is the same kernel
    assert bench.measured_traffic("halo3x3_nhwc bf16 th4 co64 w8 tuned", None) == k["bytes_per_launch"]


def test_traffic_records_of_several_plans_are_merged(tree):
    root, src = tree
    bench.write_traffic(str(src), 256, "halo3x3_nhwc bf16 th4 co64 w8")
    bench.write_traffic(str(src), 256, "igemm_nhwc_pipe_tapinner bf16 64x64 splitk=1 tuned")
    rec = json.load(open(root / "profiles" / "traffic.json"))
    assert set(rec["kernels"]) == {"halo3x3_nhwc bf16 th4 co64 w8", "igemm_nhwc_pipe_tapinner bf16 64x64 splitk=1"}
    assert rec["kernels"]["igemm_nhwc_pipe_tapinner bf16 64x64 splitk=1"]["kernel"] == GEMM
    assert bench.measured_traffic("igemm_nhwc_pipe_tapinner bf16 64x64 splitk=1", None) == (77 * 2 + 55) * 1024


def test_traffic_record_is_dropped_when_the_kernel_sources_change(tree):
    root, src = tree
    bench.write_traffic(str(src), 256, "halo3x3_nhwc bf16 th4 co64 w8")
    path = root / "profiles" / "traffic.json"
    rec = json.load(open(path))
    rec["kernels"]["halo3x3_nhwc bf16 th4 co64 w8"]["source_hash"] = "0" * 16
    json.dump(rec, open(path, "w"))
    assert bench.measured_traffic("halo3x3_nhwc bf16 th4 co64 w8", None) is None
    assert bench.measured_traffic("maxpool3x3s2", None) is None  # no record at all


def test_source_hash_covers_only_the_kernels_own_files():
    a = bench.kernel_source_hash("halo3x3_nhwc bf16 th4 co64 w8")
    b = bench.kernel_source_hash("igemm_nhwc_pipe_tapinner bf16 64x64 splitk=1")
    assert a != b and len(a) == 16
    assert bench.kernel_source_hash("halo3x3_nhwc bf16 th8 co32 w4") == a


def test_traffic_record_without_the_kernel_fails(tree):
    _, src = tree
    with pytest.raises(SystemExit):
        bench.write_traffic(str(src), 256, "stem3x3_mfma bf16")  # no stem kernel in the counter files


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
