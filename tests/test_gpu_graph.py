"""The layer forward (route, dispatch, both expert GEMMs, combine), and a training step
(that forward keeping the pre-activations, then the combine, expert and route backward),
captured once into a HIP graph and replayed: every call is a plain kernel launch on the
caller's stream (no allocation, no memset, no host synchronisation), so a replay must give
the eager call's bits.  Replays alternate two input batches copied into the captured input
buffer, with eager work and synchronisations between them."""
import pytest
import torch

import parity_gate_gemm_amd as pg
import synth
from _gpu_common import say, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, T, d, I, E, k: bf16 grouped GEMMs; MXFP8 on 128-row ring tiles; MXFP8 on the
    # 256-row tiles (persistent GEMM2, whose tile counters are cleared by a kernel each call)
    ("bf16", 300, 256, 128, 16, 4),
    ("mxfp8", 300, 512, 512, 16, 4),
    ("mxfp8", 1000, 512, 512, 8, 2),
    # NVFP4 forward: x quantized per token inside the call, fp16-MFMA GEMMs on decoded codes
    ("nvfp4", 300, 256, 128, 16, 4),
]


@pytest.mark.parametrize("dtype,T,d,I,E,k", CASES)
def test_layer_forward_replays_from_a_hip_graph(dtype, T, d, I, E, k):
    say(f"case graph {dtype} T={T} d={d} I={I} E={E} k={k}")
    wl = synth.Workload("graph", T=T, d=d, inter=I, E=E, k=k, shared=True, bias=True, dtype=dtype, seed=31)
    inp = to_device(synth.make_layer_inputs(wl, device="cpu"))
    other = to_device(synth.make_layer_inputs(wl.with_(seed=32), device="cpu"))
    if dtype == "nvfp4":   # the weight banks K-blocked once, outside the graph
        inp = pg.nvfp4_pack_inputs(inp)
    batches = [inp, dict(inp, x=other["x"], x_scale=other["x_scale"])]
    fdt = {"bf16": pg.MOE_BF16, "mxfp8": pg.MOE_MXFP8, "nvfp4": pg.MOE_NVFP4}[dtype]
    ws = pg.Workspace(T, d, E, k, I, fdt, device="cuda")
    eager = [pg.layer_forward(b, k, ws=ws) for b in batches]
    assert not torch.equal(eager[0]["y"], eager[1]["y"])

    static = dict(inp, x=inp["x"].clone(),
                  x_scale=None if inp["x_scale"] is None else inp["x_scale"].clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pg.layer_forward(static, k, ws=ws, check=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = pg.layer_forward(static, k, ws=ws, check=False)
    torch.cuda.synchronize()

    for rep in range(4):
        b = rep % 2
        static["x"].copy_(batches[b]["x"])
        if static["x_scale"] is not None:
            static["x_scale"].copy_(batches[b]["x_scale"])
        graph.replay()
        torch.cuda.synchronize()
        for name in ("ids", "weights", "offsets", "perm", "row_of", "y"):
            assert torch.equal(res[name], eager[b][name]), (rep, name)
        # eager work between the replays
        again = pg.layer_forward(batches[1 - b], k, ws=ws)
        assert torch.equal(again["y"], eager[1 - b]["y"])
    assert pg.moe_check(ws) == 0
    say("  4 replays bitwise equal to the eager calls")


TRAIN_CASES = [
    # dtype, T, d, I, E, k: the bf16 backward; the MXFP8 backward of an MXFP8 layer (its
    # data GEMMs on the 128-row ring) and of an NVFP4 layer
    ("bf16", 300, 256, 128, 16, 4),
    ("mxfp8", 300, 512, 512, 16, 4),
    ("nvfp4", 300, 256, 128, 16, 4),
]


def _outputs(fwd, bwd):
    """Every tensor a training step writes, by name (gradient dicts flattened)."""
    out = {}
    for src in (fwd, bwd):
        for n, v in src.items():
            if isinstance(v, torch.Tensor):
                out[n] = v
            elif isinstance(v, dict):
                out.update({f"{n}.{m}": t for m, t in v.items()})
    return out


@pytest.mark.parametrize("dtype,T,d,I,E,k", TRAIN_CASES)
def test_training_step_replays_from_a_hip_graph(dtype, T, d, I, E, k):
    """Forward (keeping the pre-activations) and the three backward calls captured as one
    graph: every replay writes the eager step's bits, for alternating input batches."""
    say(f"case graph training step {dtype} T={T} d={d} I={I} E={E} k={k}")
    wl = synth.Workload("graph", T=T, d=d, inter=I, E=E, k=k, shared=True, bias=True, dtype=dtype, seed=41)
    inp = to_device(synth.make_layer_inputs(wl, device="cpu"))
    other = to_device(synth.make_layer_inputs(wl.with_(seed=42), device="cpu"))
    if dtype == "nvfp4":
        inp = pg.nvfp4_pack_inputs(inp)
    if dtype != "bf16":   # the weights requantised for the MXFP8 backward, once, outside the graph
        routed = {n: inp.get(n) for n in ("w1", "w3", "w2") + pg._BANK_OPT}
        inp = dict(inp, routed_t=pg.moe_mxfp8_transpose_weights(routed),
                   shared_t=pg.moe_mxfp8_transpose_weights(inp["shared"]))
    batches = [inp, dict(inp, x=other["x"], x_scale=other["x_scale"])]
    g = torch.Generator().manual_seed(43)
    dy = torch.randn(T, d, generator=g).to(torch.bfloat16).cuda()
    fdt = {"bf16": pg.MOE_BF16, "mxfp8": pg.MOE_MXFP8, "nvfp4": pg.MOE_NVFP4}[dtype]
    ws = pg.BackwardWorkspace(T, d, E, k, I, fdt, device="cuda")

    def step(b, check=True):
        fwd = pg.layer_forward(b, k, ws=ws, save_pre=True, check=check)
        bwd = pg.layer_backward(b, k, fwd, dy, ws, pre=fwd["pre"], check=check)
        return _outputs(fwd, bwd)

    eager = [step(b) for b in batches]
    assert not torch.equal(eager[0]["dx"], eager[1]["dx"])

    static = dict(inp, x=inp["x"].clone(),
                  x_scale=None if inp["x_scale"] is None else inp["x_scale"].clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(static, check=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = step(static, check=False)
    torch.cuda.synchronize()

    for rep in range(4):
        b = rep % 2
        static["x"].copy_(batches[b]["x"])
        if static["x_scale"] is not None:
            static["x_scale"].copy_(batches[b]["x_scale"])
        graph.replay()
        torch.cuda.synchronize()
        assert set(res) == set(eager[b])
        for name, t in res.items():
            assert torch.equal(t, eager[b][name]), (rep, name)
        again = step(batches[1 - b])      # eager work between the replays
        assert torch.equal(again["dx"], eager[1 - b]["dx"])
    assert pg.moe_check(ws) == 0
    say(f"  4 replays bitwise equal to the eager steps on {len(res)} outputs")
