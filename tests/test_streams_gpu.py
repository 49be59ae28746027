"""Calls on several streams at once, and from several host threads at once, give bit for bit
the results of the same calls made one after the other on one stream: the library keeps no
state between calls, and each call's scratch is ordered on its own stream."""
import threading

import numpy as np
import pytest

import workloads
from tests.gpu_util import log, to_device

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _problems():
    """Four different calls (workload, seed, options) and their device inputs."""
    import torch
    out = []
    for i, (shape, dt, gate, zoh) in enumerate([((2, 96, 24, 20, 16, 4), "bf16", False, False),
                                                 ((1, 64, 40, 36, 16, 4), "f32", True, True),
                                                 ((3, 100, 1, 197, 16, 2), "bf16", True, False),
                                                 ((2, 70, 16, 24, 8, 4), "f32", False, True)]):
        wl = workloads.custom(*shape, dt)
        dev = to_device(workloads.make_inputs(wl, seed=60 + i), wl)
        z = None
        if gate:
            g = workloads.make_gate(wl, 60 + i)
            z = (torch.from_numpy(g["z_bf16"].view(np.int16)).view(torch.bfloat16)
                 if dt == "bf16" else torch.from_numpy(g["z"])).to("cuda:0")
        out.append((wl, dev, z, zoh))
    return out


def _call(problem, stream=None):
    import selective_scan_ss2d_amd as ss
    wl, dev, z, zoh = problem
    fn = ss.ss2d_forward_ex if wl.K == 4 else ss.ss1d_bidir_forward_ex
    return fn(*[dev[k] for k in ARGS], z=z, zoh=zoh, stream=stream)


def test_concurrent_streams_match_sequential():
    import torch
    problems = _problems()
    log("case streams: sequential reference")
    ref = [_call(p).clone() for p in problems]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in problems]
    for rnd in range(3):
        log(f"case streams: round {rnd}")
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        outs = []
        for p, s in zip(problems, streams):
            with torch.cuda.stream(s):
                outs.append(_call(p, stream=s))
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(_bits(o), _bits(r)), f"round {rnd}, call {i}"


def test_host_threads_match_sequential():
    import torch
    problems = _problems()
    log("case threads: sequential reference")
    ref = [_call(p).clone() for p in problems]
    torch.cuda.synchronize()
    results = [None] * len(problems)
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [_call(problems[i], stream=s) for _ in range(3)]
            s.synchronize()
            results[i] = outs
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    log("case threads: 4 host threads, 3 calls each")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(problems))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a host thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, outs in enumerate(results):
        for j, o in enumerate(outs):
            assert torch.equal(_bits(o), _bits(ref[i])), f"thread {i}, call {j}"
