"""Stream semantics of the C ABI on the GPU: every call enqueues its work on
the stream it is given (a user stream gives the same bits as the default
one), calls on different streams with different workspaces may run at the
same time from different host threads, and the calls hold only kernel
launches, so a HIP graph captured from them replays to the eager results.
Every comparison is bit for bit (the default backward is deterministic)."""
import sys
import threading

import pytest
import torch

import synth
import block_sparse_varlen_amd as bsa
from block_sparse_varlen_amd.runner import DeviceCase

pytestmark = pytest.mark.gpu

OUTS = ("out", "lse", "dq", "dk", "dv")


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def case_a():  # GQA with a shared pattern, causal, three sequences with ragged tails
    return synth.random_case(601, lens_q=[300, 700, 129], N1=4, N2=2, sparse_heads=2, D=128, kind="mask",
                             causal=True, density=0.6)


def case_b():  # per-q-head lists, D = 64, fp16
    return synth.random_case(602, lens_q=[513, 200], N1=2, D=64, dtype="f16", kind="idx", width=3)


def run(dc, stream=None, times=1):
    for _ in range(times):
        dc.fwd(stream=stream)
        dc.bwd(stream=stream)


def snapshot(dc):
    return {n: getattr(dc, n).clone() for n in OUTS}


def same(dc, ref, what):
    for n in OUTS:
        a, b = getattr(dc, n), ref[n]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (what, n)


def test_user_stream_matches_default_stream():
    say("streams: user stream")
    dc = DeviceCase(case_a(), with_bwd=True)
    run(dc)
    torch.cuda.synchronize()
    ref = snapshot(dc)
    for n in OUTS:
        getattr(dc, n).fill_(3.0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    run(dc, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    same(dc, ref, "user stream")


def test_concurrent_streams_from_two_threads():
    say("streams: two threads, two streams")
    cases = [DeviceCase(case_a(), with_bwd=True), DeviceCase(case_b(), with_bwd=True)]
    refs = []
    for dc in cases:
        run(dc)
        torch.cuda.synchronize()
        refs.append(snapshot(dc))
        for n in OUTS:
            getattr(dc, n).fill_(3.0)
    errors = []

    def worker(dc):
        try:
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()
            run(dc, stream=s, times=5)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(dc,)) for dc in cases]
    torch.cuda.synchronize()
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    for dc, ref in zip(cases, refs):
        same(dc, ref, dc.case.name)


def test_graph_capture_replays_to_eager_results():
    """fwd + bwd and the allocation-free forward captured into one graph each;
    several replays, with eager library work and synchronisations between
    them and the outputs overwritten before each, all give the eager bits."""
    say("streams: graph capture")
    dc = DeviceCase(case_a(), with_bwd=True)
    other = DeviceCase(case_b(), with_bwd=True)
    run(dc)
    torch.cuda.synchronize()
    ref = snapshot(dc)
    nout = torch.empty_like(dc.out)
    nlse = torch.empty_like(dc.lse)

    def noalloc():
        bsa.bsa_fwd_noalloc(dc.p, dc.q, dc.k, dc.v, dc.cu_q, dc.cu_kv, dc.seqused_kv, dc.sparse, dc.count,
                            dc.block_table, nout, nlse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture (the no-alloc scratch address is looked up here)
        run(dc)
        noalloc()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        run(dc)
    with torch.cuda.graph(g2):
        noalloc()
    torch.cuda.synchronize()
    for r in range(3):
        say(f"streams: replay {r}")
        for n in OUTS:
            getattr(dc, n).fill_(3.0)
        nout.fill_(3.0)
        nlse.fill_(3.0)
        run(other)  # eager work between replays
        torch.cuda.synchronize()
        g1.replay()
        torch.cuda.synchronize()
        same(dc, ref, f"replay {r}")
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(nout.view(torch.uint8), ref["out"].view(torch.uint8)), r
        assert torch.equal(nlse, ref["lse"]), r
