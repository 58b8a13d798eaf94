"""Host logic of bench.py (no GPU): the one-GPU guard and the conversion of
rocprofv3 FETCH_SIZE / WRITE_SIZE counters into HBM bytes per launch."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

HEADER = '"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n'


def _csv(path, counter, calib_kib, kernels):
    """A counter CSV with one calibration multiply and (dispatch, name, KiB) rows."""
    with open(path, "w") as fh:
        fh.write(HEADER)
        fh.write(f'1,"void at::native::elementwise_kernel<MulFunctor<float>>()","{counter}",{calib_kib}\n')
        for d, name, kib in kernels:
            fh.write(f'{d},"{name}","{counter}",{kib}\n')


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_scaling(tmp_path, monkeypatch):
    """FETCH_SIZE reads 256 MiB for the 512 MiB calibration copy (scale 2),
    WRITE_SIZE 512 MiB (scale 1); kernel counters are averaged per dispatch,
    converted from KiB and scaled, and keyed by the kernel's source hash."""
    fwd = "void bsa::(anonymous namespace)::k_fwd<bsa::BF16, 128, false, false>(bsa::FwdArgs)"
    pre = "void bsa::(anonymous namespace)::k_bwd_pre<bsa::BF16, 128>(bsa::BwdPreArgs)"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # two dispatches of the forward (counter rows of several instances add up)
    _csv(fetch, "FETCH_SIZE", 262144, [(2, fwd, 600), (2, fwd, 400), (3, fwd, 1000), (4, pre, 50)])
    _csv(write, "WRITE_SIZE", 524288, [(2, fwd, 500), (3, fwd, 500), (4, pre, 8)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.write_traffic(str(fetch), str(write))
    t = json.loads(out.read_text())
    assert t["_fetch_scale"] == 2.0 and t["_write_scale"] == 1.0
    assert t["fwd"]["fetch_bytes"] == 1000 * 1024 * 2
    assert t["fwd"]["write_bytes"] == 500 * 1024
    assert t["fwd"]["bytes_per_launch"] == 1000 * 1024 * 2 + 500 * 1024
    assert t["fwd"]["source_sha"] == bench.kernel_source_sha("fwd")
    assert t["bwd_pre"]["bytes_per_launch"] == 50 * 1024 * 2 + 8 * 1024
    assert "source_sha" not in t["bwd_pre"]


def test_profiler_detection(monkeypatch):
    """Under rocprofv3 (its ROCPROF* environment or its preloaded tool
    library) the bench spawns nothing: no clock sampling, no oracle pool."""
    for k in list(os.environ):
        if k.startswith("ROCPROF"):
            monkeypatch.delenv(k)
    monkeypatch.setenv("LD_PRELOAD", "")
    assert not bench.under_profiler()
    monkeypatch.setenv("ROCPROF_OUTPUT_PATH", "/tmp/x")
    assert bench.under_profiler()
    monkeypatch.delenv("ROCPROF_OUTPUT_PATH")
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/rocprofiler-sdk/librocprofiler-sdk-tool.so")
    assert bench.under_profiler()


def test_step_statistics():
    st = bench.stats_ms([3.0, 1.0, 2.0, 10.0, 4.0])
    assert st["median"] == 3.0 and st["min"] == 1.0 and st["mean"] == 4.0
    assert 4.0 < st["p90"] <= 10.0


def test_cpu_workers_bounded():
    assert 1 <= bench.cpu_workers() <= 16
    assert isinstance(bench.cpu_model(), str)
