"""Host logic of bench.py (no GPU): the algorithmic work it divides by, the
counter-record bookkeeping behind roofline.traffic, and the one-GPU guard.

The expected byte and FLOP counts are written out from the definitions the
roofline uses, not from bench.py: a producer moves its inputs once and its
outputs once (AdaRMS: residual, x and the residual output in bf16, the FP8
codes, the gate row or per-element gate, the three modulation rows;
per-token table: x in bf16, two fp32 chunks of the per-token conditioning,
two fp32 table rows, the codes); a GEMM moves X8 + W8 + the bf16 output
(+ the bf16 bias) and does 2 M N K FLOPs.
"""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _packs(w):
    return [{"splits": g, "bias": (object() if w.bias else None)} for g in w.gemms]


@pytest.mark.parametrize("cid,kind,rows,nbytes,flops", [
    # AdaRMS, 16 x 512: 3*2*16*512 + 16*512 + 512*2 + 3*512*2
    (1, "norm1", 16, 61_440, 0),
    # QKV 16 x 768 x 512: 16*512 + 768*512 + 16*768*2
    (1, "gemm1", 16, 425_984, 2 * 16 * 768 * 512),
    # AdaRMS, 256 x 2048, broadcast gate (both sites)
    (2, "norm1", 256, 3_686_400, 0),
    (2, "norm2", 256, 3_686_400, 0),
    # QKV 256 x 2560 x 2048 and gate/up 256 x 16384 x 2048
    (2, "gemm1", 256, 7_077_888, 2 * 256 * 2560 * 2048),
    (2, "gemm2", 256, 42_467_328, 2 * 256 * 16384 * 2048),
    # per-token table, 8192 x 3072: 2*R*D + 4*R*D + 2*D*4 + R*D
    (3, "norm1", 8192, 176_185_344, 0),
    # QKV + bias 8192 x 9216 x 3072: 8192*3072 + 9216*3072 + 8192*9216*2 + 9216*2
    (3, "gemm1", 8192, 204_490_752, 2 * 8192 * 9216 * 3072),
    # AdaRMS, 64 x 4096 with a per-element gate (64*4096*2 gate bytes)
    (4, "norm1", 64, 2_383_872, 0),
    # QKV 64 x 6144 x 4096 and at one row
    (4, "gemm1", 64, 26_214_400, 2 * 64 * 6144 * 4096),
    (4, "gemm1", 1, 25_182_208, 2 * 1 * 6144 * 4096),
    # per-token table, 2048 x 16384; gate/up 2048 x 32768 x 16384
    (5, "norm1", 2048, 235_012_096, 0),
    (5, "gemm1", 2048, 704_643_072, 2 * 2048 * 32768 * 16384),
])
def test_algorithmic_work(cid, kind, rows, nbytes, flops):
    w = wl.WORKLOADS[cid]
    b, f = bench.kernel_work(w, kind, rows, _packs(w))
    assert int(b) == nbytes
    assert int(f) == flops


def _write_counter_csv(folder, rows):
    """A rocprofv3 --pmc csv folder with (dispatch, kernel, counter, value) rows."""
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for d, k, c, v in rows:
            wr.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_summarize_pmc_scales_by_the_copy(tmp_path, monkeypatch):
    """The record takes the median of the last --launches dispatches of the
    kernel (earlier set-up dispatches of it are ignored) and scales each
    counter by true bytes / what the counter reads for the plain copy."""
    gemm = "void frt::gemm_kernel<...>"
    copy = "__amd_rocclr_copyBuffer"
    kib = bench.COPY_BYTES / 1024
    f, wdir, cf, cw = (str(tmp_path / n) for n in ("f", "w", "cf", "cw"))
    # one set-up dispatch (ignored), then three profiled ones
    _write_counter_csv(f, [(1, gemm, "FETCH_SIZE", 99999.0)] +
                       [(2 + i, gemm, "FETCH_SIZE", v) for i, v in enumerate([1000.0, 1010.0, 990.0])])
    _write_counter_csv(wdir, [(1, gemm, "WRITE_SIZE", 5.0)] +
                       [(2 + i, gemm, "WRITE_SIZE", 400.0) for i in range(3)])
    # the copy: FETCH_SIZE reads half the true bytes, WRITE_SIZE all of them
    _write_counter_csv(cf, [(i, copy, "FETCH_SIZE", kib / 2) for i in range(3)])
    _write_counter_csv(cw, [(i, copy, "WRITE_SIZE", kib) for i in range(3)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    a = SimpleNamespace(summarize_pmc=[f, wdir, cf, cw], profile_kernel="gemm2", launches=3, workload=2)
    bench.summarize_pmc(a)
    rec = json.load(open(tmp_path / "profiles" / "traffic_w2_gemm2.json"))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes"] == 1000 * 1024 * 2
    assert rec["write_bytes"] == 400 * 1024
    assert rec["traffic_bytes"] == 1000 * 1024 * 2 + 400 * 1024
    assert rec["sources_sha256"] == bench.kernel_sources_sha("gemm2")


def test_summarize_pmc_sums_the_launches_of_one_call(tmp_path, monkeypatch):
    """A GEMM call made of two launches (a 256x256 head, then a 256x128 tail)
    counts as one call: its two dispatches are summed, and the median runs
    over calls, not over a mixture of head and tail dispatches."""
    head = "void frt::gemm256_kernel<false, false, false, 256>(frt::GemmArgs)"
    tail = "void frt::gemm256_kernel<false, false, false, 128>(frt::GemmArgs)"
    copy = "__amd_rocclr_copyBuffer"
    kib = bench.COPY_BYTES / 1024
    f, wdir, cf, cw = (str(tmp_path / n) for n in ("f", "w", "cf", "cw"))
    seq = [(head, 900.0), (tail, 100.0)] * 4   # a set-up call, then three profiled ones
    _write_counter_csv(f, [(i, k, "FETCH_SIZE", v) for i, (k, v) in enumerate(seq)])
    _write_counter_csv(wdir, [(i, k, "WRITE_SIZE", v / 2) for i, (k, v) in enumerate(seq)])
    _write_counter_csv(cf, [(i, copy, "FETCH_SIZE", kib) for i in range(3)])
    _write_counter_csv(cw, [(i, copy, "WRITE_SIZE", kib) for i in range(3)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    a = SimpleNamespace(summarize_pmc=[f, wdir, cf, cw], profile_kernel="gemm1", launches=3, workload=3)
    bench.summarize_pmc(a)
    rec = json.load(open(tmp_path / "profiles" / "traffic_w3_gemm1.json"))
    assert rec["calls"] == [3, 3]
    assert rec["fetch_bytes"] == 1000 * 1024 and rec["write_bytes"] == 500 * 1024


def test_traffic_record_needs_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.load_traffic(2, "gemm2") is None            # no record
    rec = {"traffic_bytes": 123, "sources_sha256": bench.kernel_sources_sha("gemm2")}
    (tmp_path / "traffic_w2_gemm2.json").write_text(json.dumps(rec))
    assert bench.load_traffic(2, "gemm2") == 123
    monkeypatch.setattr(bench, "kernel_sources_sha", lambda kind=None: "0" * 64)
    assert bench.load_traffic(2, "gemm2") is None            # kernels changed


def test_traffic_record_follows_its_own_kernel_sources():
    """A GEMM record covers the GEMM's sources, a producer record the
    producer's: a change to one kernel file leaves the other's hash alone."""
    g = set(bench._kernel_files("gemm1")[1])
    n = set(bench._kernel_files("norm1")[1])
    assert {"frt_gemm.hip", "frt_gemm_epilogue.inc"} <= g and "frt_norm.hip" not in g
    assert "frt_norm.hip" in n and "frt_gemm.hip" not in n
    assert {"frt_api.hip", "frt_device.h", "frt_internal.h"} <= g & n
    assert bench.kernel_sources_sha("gemm1") != bench.kernel_sources_sha("norm1")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
