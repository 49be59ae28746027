"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph on ROCm): a call's
stream-ordered scratch becomes an allocation of the graph, and every replay gives, bit for
bit, the eager call's outputs.  Each graph is replayed several times, with the outputs
overwritten by eager kernels and the device synchronised between the replays."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import log, to_device

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
REPLAYS = 4


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check_replays(what, call):
    """call() -> dict of output tensors.  Eager reference first, then capture and replays."""
    import torch
    log(f"case graph {what}")
    eager = {k: v.clone() for k, v in call().items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up call on a side stream, as capture requires
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = call()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for t in outs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, ref in eager.items():
            assert torch.equal(_bits(outs[k]), _bits(ref)), f"{what}: replay {r}, output {k}"
    del graph


def _inputs(wl, seed):
    import torch
    inp = workloads.make_inputs(wl, seed=seed)
    dev = to_device(inp, wl)

    def image(g, key):
        if wl.dtype == "bf16":
            return torch.from_numpy(g[key + "_bf16"].view(np.int16)).view(torch.bfloat16).to(
                "cuda:0")
        return torch.from_numpy(g[key]).to("cuda:0")
    z = image(workloads.make_gate(wl, seed), "z")
    dy = image(workloads.make_output_grad(wl, seed), "dy")
    return dev, z, dy


@pytest.mark.parametrize("case", [(2, 96, 24, 20, 16, "bf16"), (1, 64, 40, 36, 16, "f32")],
                         ids=["one_pass_bf16", "chunked_f32"])
def test_forward_in_graph(case):
    import selective_scan_ss2d_amd as ss
    B, D, H, W, N, dt = case
    wl = workloads.custom(B, D, H, W, N, 4, dt)
    dev, z, _ = _inputs(wl, 51)
    args = [dev[k] for k in ARGS]
    _check_replays(f"forward {case}", lambda: {"y": ss.ss2d_forward(*args)})
    _check_replays(f"forward gate+zoh {case}",
                   lambda: {"y": ss.ss2d_forward_ex(*args, z=z, zoh=True)})


def test_bidir_forward_in_graph():
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(3, 100, 1, 197, 16, 2, "bf16")
    dev, z, _ = _inputs(wl, 52)
    args = [dev[k] for k in ARGS]
    _check_replays("bidir forward gated", lambda: {"y": ss.ss1d_bidir_forward_ex(*args, z=z)})


@pytest.mark.parametrize("gate,zoh", [(False, False), (True, True)], ids=["plain", "gate_zoh"])
def test_backward_in_graph(gate, zoh):
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 70, 16, 24, 16, 4, "bf16")
    dev, z, dy = _inputs(wl, 53)
    args = [dev[k] for k in ARGS]
    _check_replays(f"backward gate={gate} zoh={zoh}",
                   lambda: ss.ss2d_backward_ex(*args, dy, z=z if gate else None, zoh=zoh))


def test_front_chain_in_graph():
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 64, 12, 16, 16, 4, "bf16")
    dev, z, _ = _inputs(wl, 54)
    w = workloads.make_front_weights(wl, 54, R=2, KW=4)
    fw = [torch.from_numpy(w[k]).to("cuda:0") for k in ("conv_w", "conv_b", "x_proj_w",
                                                        "dt_proj_w")]

    def chain():
        o = ss.ss2d_project(dev["x"], *fw)
        y = ss.ss2d_forward_routes(o["u"], o["dt_raw"], dev["A_log"], o["Bs"], o["Cs"],
                                   dev["Ds"], dev["dt_bias"], wl.H, wl.W, z=z)
        return {"y": y, **o}
    _check_replays("front end + routes operator", chain)


@pytest.mark.parametrize("gate", [False, True], ids=["plain", "gate"])
def test_training_pair_in_graph(gate):
    """The training forward and the backward from its kept state, captured as one graph."""
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 70, 16, 24, 16, 4, "bf16")
    dev, z, dy = _inputs(wl, 55)
    args = [dev[k] for k in ARGS]
    zz = z if gate else None
    saved = torch.empty(ss.saved_state_bytes(4, wl.B, wl.D, wl.H * wl.W, wl.N, gate) // 4,
                        dtype=torch.float32, device="cuda:0")

    def step():
        y, _ = ss.ss2d_forward_save(*args, z=zz, saved=saved)
        return {"y": y, **ss.ss2d_backward_saved(*args, dy, saved, z=zz)}
    _check_replays(f"training pair gate={gate}", step)
