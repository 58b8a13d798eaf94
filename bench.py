"""Throughput of block-sparse varlen attention (forward + backward) on one
MI355X.

Workload: the long-context block-sparse case -- 2 sequences x 16384 tokens,
16 q/kv heads, D = 128, bf16, 128x128 blocks, a block-causal mask keeping the
diagonal, the 4 preceding and 8 random earlier blocks per q-block.  One step
= one training step's attention: bsa_build_index (with the transposed lists)
once, then bsa_fwd and bsa_bwd on that index (BSA_FLAG_INDEX_BUILT), inputs
resident in HBM.  The line also carries each call timed on its own with its
own index build inside (the unit the per-pass fractions are quoted on).
FLOPs are counted over the selected blocks only: 4 r c D per visited
(q-head, q-block, kv-block) pair forward and 10 r c D backward (r, c = valid
rows / columns of the pair).

Prints one JSON line.  ``--gpus`` above 1 is refused: the benchmark runs on one
GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
METRIC = "fwd & bwd TFLOP/s over selected blocks; % of MI355X bf16 MFMA peak"
WORKLOAD = "long-context block-sparse fwd+bwd: TND 2x16384, N1=N2=16, D=128, bf16, 128x128 blocks, " \
           "block-causal mask (diagonal + 4 preceding + 8 random earlier blocks per q-block)"
# other workloads for --workload (not the default line): the rest of the
# benchmark configurations, run fwd + bwd
OTHER_WORKLOADS = {
    1: "tiny fwd+bwd: TND, 1 x 512 tokens, N1=N2=2, D=64, fp16, 128x128 blocks, Bernoulli(0.5) block mask "
       "with the diagonal kept",
    2: "dense varlen causal fwd+bwd: TND, B=4, lengths U{512..4096}, N=16, D=128, bf16, all blocks",
    3: "sabi block-sparse prefill fwd+bwd: B=1, N=32, S=32768, D=128, bf16, block (128,512), keep U{1..16}",
    4: "GQA + paged-KV block-sparse fwd+bwd: B=8, lengths U{1024..8192}, N1=32, N2=8, D=128, bf16, "
       "128-token pages, idx top-16 (counts U{4..16}), causal",
    6: "per-token selection fwd+bwd (block shape [1, 128]): TND 2 x 4096, N1=32, N2=8, D=128, bf16, "
       "idx top-16 per query token (counts U{4..16}), causal",
}
# GEMMs each kernel performs out of the counted ones: fwd = QK^T, PV (4 r c D);
# dK/dV kernel = S, dP, dV, dK (8 r c D); dQ kernel = dQ (2 r c D; its
# recomputation of S and dP is not counted).
ALG_FLOPS_PER_RCD = {"fwd": 4, "bwd_dkdv": 8, "bwd_dq": 2}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_cfg5.json")
KERNEL_SOURCES = {
    "fwd": ["bsa_fwd.hip", "bsa_attn.h", "bsa_device.h", "bsa_internal.h"],
    "bwd_dkdv": ["bsa_bwd.hip", "bsa_attn.h", "bsa_device.h", "bsa_internal.h"],
    "bwd_dq": ["bsa_bwd.hip", "bsa_attn.h", "bsa_device.h", "bsa_internal.h"],
}


def kernel_source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "block_sparse_varlen_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def visited_rcd(case, idx):
    """Sum over visited (q-head, q-block, kv-block) pairs of r * c * D."""
    lens_q = np.diff(case.cu_q)
    lens_kv = case.seqused_kv if case.paged else np.diff(case.cu_kv)
    nqb = -(-lens_q // case.bx)
    qbase = np.concatenate([[0], np.cumsum(nqb)])
    TQB, R = idx["TQB"], idx["R"]
    rp, cols = idx["row_ptr"], idx["cols"]
    hpr = 1 if case.sparse_heads == case.N1 else case.N1 // case.N2
    total = 0
    for r in range(R):
        qg = r % TQB
        b = int(np.searchsorted(qbase, qg, side="right") - 1)
        qb = qg - int(qbase[b])
        rows = min(case.bx, int(lens_q[b]) - qb * case.bx)
        kb = cols[rp[r]:rp[r + 1]].astype(np.int64)
        c = np.minimum(case.by, int(lens_kv[b]) - kb * case.by)
        total += rows * int(c.sum())
    return total * hpr * case.D


def cpu_model() -> str:
    """The host CPU's model name, read from /proc/cpuinfo (no subprocess)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers() -> int:
    """Worker processes for the oracle baseline: the CPUs this process may run
    on, at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_CPU_CASE = None  # the workload, inherited by the forked oracle workers


def _cpu_unit_rcd(case, idx, qbase, b, h, qb):
    lens_q = np.diff(case.cu_q)
    rp = idx["row_ptr"]
    r = h * idx["TQB"] + int(qbase[b]) + qb
    rows = min(case.bx, int(lens_q[b]) - qb * case.bx)
    kbs = idx["cols"][rp[r]:rp[r + 1]]
    c = np.minimum(case.by, int(np.diff(case.cu_kv)[b]) - kbs * case.by).sum()
    return rows * int(c) * case.D


def _cpu_worker(arg):
    """One oracle worker: whole (sequence, q-head, q-block) units, forward and
    backward each, drawn at random until the deadline; one BLAS thread."""
    seed, deadline = arg
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    case = _CPU_CASE
    lens_q = np.diff(case.cu_q)
    nqb = -(-lens_q // case.bx)
    qbase = np.concatenate([[0], np.cumsum(nqb)])
    idx = oracle.index_products(case, with_csc=False)
    rng = np.random.default_rng(seed)
    done, flops = 0, 0.0
    while time.time() < deadline:
        b = int(rng.integers(case.B))
        h = int(rng.integers(case.N1))
        qb = int(rng.integers(nqb[b]))
        oracle.forward(case, sample=[(b, h, qb)])
        oracle.backward(case, sample_rows=[(b, h, qb)])
        flops += 14.0 * _cpu_unit_rcd(case, idx, qbase, b, h, qb)
        done += 1
    return done, flops


def cpu_baseline(case, budget_s: float):
    """The CPU oracle, as it stands, on random (sequence, q-head, q-block)
    units of the same workload (forward + backward each), run by a pool of
    forked worker processes with one BLAS thread each for about ``budget_s``
    seconds.  Called before the process touches the GPU, so the workers fork
    from a process without GPU state and nothing is exec'd."""
    import multiprocessing

    global _CPU_CASE
    _CPU_CASE = case
    n = cpu_workers()
    ctx = multiprocessing.get_context("fork")
    t0 = time.time()
    with ctx.Pool(n) as pool:
        res = pool.map(_cpu_worker, [(1000 + i, t0 + budget_s) for i in range(n)])
    dt = time.time() - t0
    _CPU_CASE = None
    done = sum(r[0] for r in res)
    flops = sum(r[1] for r in res)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": n, "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"{done} random (sequence, q-head, q-block) units of the same workload, fwd+bwd each, "
                      f"{dt:.1f} s of fp64 NumPy over {n} worker processes (1 BLAS thread each)"}


def under_profiler() -> bool:
    """True inside a rocprofv3 run (its environment or preloaded tool
    library): nothing may be spawned there, as the profiler's preload would
    follow the child."""
    if any(k.startswith("ROCPROF") for k in os.environ):
        return True
    return "rocprof" in os.environ.get("LD_PRELOAD", "")


def stats_ms(xs):
    xs = np.sort(np.asarray(xs, dtype=np.float64))
    return {"median": round(float(np.median(xs)), 4), "min": round(float(xs[0]), 4),
            "p90": round(float(np.percentile(xs, 90)), 4), "mean": round(float(xs.mean()), 4)}


# bench kernel keys by the HIP kernel names rocprofv3 reports
KERNEL_KEYS = {"k_fwd<": "fwd", "k_bwd_dkdv<": "bwd_dkdv", "k_bwd_dq<": "bwd_dq", "k_bwd_pre<": "bwd_pre"}
CALIB_BYTES = 512 << 20  # --calib-copy: y = x * 1 over 512 MiB of fp32 (reads and writes that much)


def short_kernel_name(name: str) -> str:
    """A rocprofv3 kernel name without namespaces and arguments."""
    n = name.replace("void ", "").replace("bsa::(anonymous namespace)::", "").replace("bsa::", "")
    return n.split("(")[0]


def write_traffic(fetch_csv: str, write_csv: str, out_path: str = None) -> None:
    """Per-launch HBM bytes of each kernel from two rocprofv3 --pmc runs of
    ``bench.py --calib-copy`` (FETCH_SIZE, then WRITE_SIZE, in KiB per
    dispatch).  Each counter is scaled by bytes / counter of the calibration
    multiply, whose traffic is known.  Writes ``out_path`` (default
    TRAFFIC_FILE): the attention kernels under the bench's keys, with the hash
    of each kernel's sources so that a later change of a kernel invalidates
    its entry, and every kernel under its own name."""
    import csv

    def per_dispatch(path, counter):
        tot, disp = {}, {}
        calib = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "MulFunctor" in name:
                calib.append(v)
                continue
            keys = [key for pat, key in KERNEL_KEYS.items() if pat in name]
            if not keys and "bsa::" in name:
                keys = ["kernel:" + short_kernel_name(name)]
            for key in keys:
                tot[key] = tot.get(key, 0.0) + v
                disp.setdefault(key, set()).add(r["Dispatch_Id"])
        if not calib:
            raise SystemExit(f"{path}: no calibration multiply found (run bench.py with --calib-copy)")
        scale = CALIB_BYTES / (sum(calib) / len(calib) * 1024.0)
        return {k: tot[k] / len(disp[k]) * 1024.0 * scale for k in tot}, scale

    fetch, fs = per_dispatch(fetch_csv, "FETCH_SIZE")
    write, ws = per_dispatch(write_csv, "WRITE_SIZE")
    out = {"_note": "HBM bytes per launch = FETCH_SIZE * fetch_scale + WRITE_SIZE * write_scale (counters in KiB; "
                    "scales from a 512 MiB copy)", "_fetch_scale": fs, "_write_scale": ws}
    for k in sorted(set(fetch) & set(write)):
        ent = {"fetch_bytes": round(fetch[k]), "write_bytes": round(write[k]),
               "bytes_per_launch": round(fetch[k] + write[k])}
        if k in KERNEL_SOURCES:
            ent["source_sha"] = kernel_source_sha(k)
        out[k] = ent
    with open(out_path or TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def sample_sclk(step, seconds: float = 3.0):
    """Average graphics clock (MHz) over the XCDs, read with ``amd-smi metric
    --clock`` from a second thread while ``step`` runs back to back for about
    ``seconds``; None when the tool is missing or prints no clock."""
    import re
    import subprocess
    import threading

    import torch

    samples = []
    stop = threading.Event()

    def sampler():
        time.sleep(0.5)
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock"], capture_output=True, text=True,
                                   timeout=10)
            except (OSError, subprocess.SubprocessError):
                return
            clks = [int(m) for m in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", r.stdout)]
            if clks:
                samples.append(sum(clks) / len(clks))
            time.sleep(0.1)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(20):
            step()
    torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    return (sum(samples) / len(samples), len(samples)) if samples else (None, 0)


PEAK_FP8_TFLOPS = 2 * 2516.6  # MI355X dense fp8 MFMA


def fp8_main(args, case, workload):
    """Forward only with FLOAT8_E4M3 q / k / v and bf16 output (the pages'
    quantType 5): a step is the block index build (no transposed lists) plus
    one forward call.  Prints one JSON line."""
    import torch
    import synth
    import block_sparse_varlen_amd as bsa
    from block_sparse_varlen_amd.runner import DeviceCase

    case = synth.to_fp8(case, "bf16")
    dc = DeviceCase(case, with_bwd=False)
    idx = dc.index(False)
    f_fwd = 4.0 * visited_rcd(case, idx)
    stream = torch.cuda.current_stream()

    def step():
        dc.build_index(False)
        dc.fwd(prebuilt=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    bsa.bsa_profile_enable(True)
    bsa.bsa_profile_reset()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    per_kernel = {}
    for kid, name in bsa.KERNEL_NAMES.items():
        n, tot = bsa.bsa_profile_read(kid)
        if n:
            per_kernel[name] = tot / n
    bsa.bsa_profile_enable(False)
    achieved = f_fwd / (per_kernel["fwd"] * 1e-3) / 1e12
    value = f_fwd / (ms_step * 1e-3) / 1e12
    line = {
        "metric": "fwd TFLOP/s over selected blocks, e4m3 q/k/v (quantType 5); % of MI355X fp8 MFMA peak",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (P e4m3, fp32 softmax, bf16 out)",
        "data": "synthetic (seeded N(0,1) Q/K/V rounded to e4m3, seeded block selection)",
        "config": {"workload": workload + ", forward only in e4m3"},
        "frac_of_peak": round(value / PEAK_FP8_TFLOPS, 4),
        "kernels_ms": {k: round(v, 4) for k, v in per_kernel.items()},
        "roofline": {"kernel": "fwd", "bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    if len(sys.argv) in (4, 5) and sys.argv[1] == "--write-traffic":
        write_traffic(*sys.argv[2:])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5, 6],
                    help="benchmark configuration (default 5, the long-context workload the metric is quoted on; "
                         "6 = per-token selection, a measurement beside them)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the graphics clock (always skipped under a profiler)")
    ap.add_argument("--fp8", action="store_true",
                    help="forward only with e4m3 q/k/v and bf16 output (a separate line; not the default metric)")
    ap.add_argument("--self-index", action="store_true",
                    help="the step lets bsa_fwd and bsa_bwd each build their own block index (no shared build)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 512 MiB elementwise copy (reference for HBM byte counters)")
    ap.add_argument("--dq-atomic", action="store_true",
                    help="backward with dQ by fp32 atomics inside the dK/dV kernel (BSA_FLAG_DQ_ATOMIC)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    profiled = under_profiler()
    if profiled:
        args.no_clock = True
        args.no_cpu_baseline = True

    import torch
    import synth

    print("bench: generating inputs", file=sys.stderr, flush=True)
    workload = WORKLOAD if args.workload == 5 else OTHER_WORKLOADS[args.workload]
    if args.fp8:
        import block_sparse_varlen_amd  # noqa: F401  (fails loudly without the library)
        torch.cuda.set_device(0)
        fp8_main(args, synth.CONFIGS[args.workload](), workload)
        return
    if args.workload in synth.EXTRA:
        case = synth.EXTRA[args.workload]()
    elif args.workload in (3, 4):
        case = synth.CONFIGS[args.workload](with_dout=True)
    else:
        case = synth.CONFIGS[args.workload]()
    cpu = None
    if not args.no_cpu_baseline:
        # before the GPU is touched: the oracle workers fork from this process
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(case, args.cpu_budget)

    import block_sparse_varlen_amd as bsa
    from block_sparse_varlen_amd.runner import DeviceCase

    torch.cuda.set_device(0)
    dc = DeviceCase(case, with_bwd=True, flags=bsa.BSA_FLAG_DQ_ATOMIC if args.dq_atomic else 0)
    idx = dc.index(False)
    rcd = visited_rcd(case, idx)
    f_fwd, f_bwd = 4.0 * rcd, 10.0 * rcd
    stream = torch.cuda.current_stream()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # one training step: the block index is built once (bsa_build_index, with
    # the transposed lists) and both passes run on it (BSA_FLAG_INDEX_BUILT)
    shared = not args.self_index

    def step():
        if shared:
            dc.build_index(True)
        dc.fwd(prebuilt=shared)
        dc.bwd(prebuilt=shared)

    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step timing (HIP events on the launch stream): the K steps as one
    # bracket, and each step's own bracket for the median / min / p90
    print("bench: timed steps", file=sys.stderr, flush=True)
    ev = [(E(), E()) for _ in range(args.steps)]
    e0, e1 = E(), E()
    torch.cuda.synchronize()
    e0.record(stream)
    for k in range(args.steps):
        ev[k][0].record(stream)
        step()
        ev[k][1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    step_stats = stats_ms([a.elapsed_time(b) for a, b in ev])

    # split of the shared-index step: index build, forward call, backward call
    # -- events between the calls of back-to-back steps, one synchronisation
    # at the end, so no bracket starts on an idle GPU
    ev = [[E() for _ in range(4)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record(stream)
        dc.build_index(True)
        ev[k][1].record(stream)
        dc.fwd(prebuilt=True)
        ev[k][2].record(stream)
        dc.bwd(prebuilt=True)
        ev[k][3].record(stream)
    torch.cuda.synchronize()
    idx_st = stats_ms([e[0].elapsed_time(e[1]) for e in ev])
    fwd_st = stats_ms([e[1].elapsed_time(e[2]) for e in ev])
    bwd_st = stats_ms([e[2].elapsed_time(e[3]) for e in ev])

    # each call on its own, building its own index inside (the unit the
    # per-pass fractions are quoted on)
    ev = [[E() for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record(stream)
        dc.fwd()
        ev[k][1].record(stream)
        dc.bwd()
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    fwd_call = stats_ms([e[0].elapsed_time(e[1]) for e in ev])
    bwd_call = stats_ms([e[1].elapsed_time(e[2]) for e in ev])

    # per-kernel durations from events the library records around its launches
    bsa.bsa_profile_enable(True)
    bsa.bsa_profile_reset()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    per_kernel = {}
    for kid, name in bsa.KERNEL_NAMES.items():
        n, tot = bsa.bsa_profile_read(kid)
        if n:
            per_kernel[name] = {"launches": n, "avg_ms": tot / n}
    bsa.bsa_profile_enable(False)
    print("bench: per-kernel " + json.dumps(per_kernel), file=sys.stderr, flush=True)

    sclk, nsamp = (None, 0)
    if not args.no_clock:
        print("bench: sampling the graphics clock", file=sys.stderr, flush=True)
        sclk, nsamp = sample_sclk(step)

    if args.calib_copy:
        x = torch.ones(128 << 20, dtype=torch.float32, device="cuda")  # 512 MiB
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        del x, y

    # with atomic dQ the dK/dV kernel also does the dQ GEMM, and the "dQ" launch
    # is the fp32 -> dtype conversion
    alg_per_rcd = dict(ALG_FLOPS_PER_RCD, bwd_dkdv=10, bwd_dq=0) if args.dq_atomic else ALG_FLOPS_PER_RCD
    dominant = max((k for k in per_kernel if alg_per_rcd.get(k)), key=lambda k: per_kernel[k]["avg_ms"])
    alg = alg_per_rcd[dominant] * rcd
    achieved = alg / (per_kernel[dominant]["avg_ms"] * 1e-3) / 1e12
    traffic = None
    if args.workload == 5 and not args.dq_atomic and os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        ent = tr.get(dominant)
        if ent and ent.get("source_sha") == kernel_source_sha(dominant):
            traffic = ent.get("bytes_per_launch")

    def rate(flops, ms):
        t = flops / (ms * 1e-3) / 1e12
        return {"tflops": round(t, 3), "frac_of_peak": round(t / PEAK_BF16_TFLOPS, 4)}

    total_tflops = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(total_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f16": "fp16"}[case.dtype],
        "data": "synthetic (seeded N(0,1) Q/K/V/dO, seeded block selection)",
        "config": {"workload": workload + (", dQ by fp32 atomics" if args.dq_atomic else ""),
                   "global_batch": case.B, "seq_len": int(np.diff(case.cu_q).max()),
                   "heads": case.N1, "head_dim": case.D, "block_shape": [case.bx, case.by],
                   "parallelism": "single GPU"},
        "frac_of_peak": round(total_tflops / PEAK_BF16_TFLOPS, 4),
        "step_ms": step_stats,
        # each call on its own, its own index build inside (median over the
        # timed iterations): the per-pass rates
        "fwd_call": dict(ms=fwd_call, flops=f_fwd, **rate(f_fwd, fwd_call["median"])),
        "bwd_call": dict(ms=bwd_call, flops=f_bwd, **rate(f_bwd, bwd_call["median"])),
        # the shared-index step split into its three brackets (medians)
        "index": {"ms": idx_st},
        "fwd": dict(ms=fwd_st, **rate(f_fwd, fwd_st["median"])),
        "bwd": dict(ms=bwd_st, **rate(f_bwd, bwd_st["median"])),
        "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in per_kernel.items()},
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        # the clock the steps actually ran at (the peak assumes 2.4 GHz), and the
        # step's fraction of the peak scaled to that clock
        "clock": {"sclk_mhz": round(sclk, 1) if sclk else None, "samples": nsamp,
                  "method": "amd-smi metric --clock, mean over XCDs, while steps run back to back",
                  "frac_of_peak_at_sclk": round(total_tflops / (PEAK_BF16_TFLOPS * sclk / 2400.0), 4) if sclk else None},
        "cpu_baseline": cpu,
    }
    if case.causal and case.sparse_kind == "none" and case.band is None:
        # dense causal: the token-exact count 4 D N1 sum_b Sq_b (Sq_b + 1) / 2 beside
        # the per-visited-block one (diagonal blocks counted whole)
        sq = np.diff(case.cu_q).astype(np.float64)
        fe = 4.0 * case.D * case.N1 * float((sq * (sq + 1) / 2).sum())
        line["causal_exact"] = {"fwd_flops": fe, "bwd_flops": 2.5 * fe,
                                "step_tflops": round(3.5 * fe / (ms_step * 1e-3) / 1e12, 3),
                                "fwd_call_tflops": round(fe / (fwd_call["median"] * 1e-3) / 1e12, 3),
                                "bwd_call_tflops": round(2.5 * fe / (bwd_call["median"] * 1e-3) / 1e12, 3)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
