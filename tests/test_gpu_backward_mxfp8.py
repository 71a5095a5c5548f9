"""GPU parity of the MXFP8 layer's backward pass against the oracle's MXFP8 backward.

The oracle applies the same readings as the library (every backward GEMM operand in
MXFP8 blocked along that GEMM's reduction dimension, the forward's h quantised per row,
the expert-output gradient in bf16) and computes every product and sum exactly in
float64, so the GPU differs from it only by fp32 accumulation and by the rare E4M3
rounding decision that such a difference flips.  Every gradient is compared as a whole
tensor, normwise (max |err| / max |ref|), to 6e-2, the MXFP8 bar: one flipped E4M3 code
moves a product by an eighth of its size, and a weight gradient summed over a few dozen
rows keeps much of that in its largest elements.  The relative Frobenius error, which
such isolated flips barely move, must stay below 1e-2.  Also checked: the requantised weights are
bit-exact against the oracle's quantiser; saved and recomputed pre-activations give the
same bits; the backward is bitwise repeatable; a token's dx does not depend on the
batch; at full size (T = 4096, d = 7168, I = 2048) the shared expert's gradients over
all tokens and one routed expert's, against the oracle's expert backward.
"""
import numpy as np
import pytest
import torch

import oracle
import parity_gate_gemm_amd as pg
import synth
from _gpu_common import LazyExperts, host, say, shared_of, to_device, values

pytestmark = pytest.mark.gpu

BAR = 6e-2        # normwise, the MXFP8 bar
BAR_FRO = 1e-2    # relative Frobenius


def _errs(got, ref):
    """(normwise max-abs-rel, relative Frobenius) error of got against ref."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    fro = np.linalg.norm(ref)
    return (float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0)),
            float(np.linalg.norm(got - ref) / (fro if fro > 0 else 1.0)))


def _check(errs):
    say("  " + ", ".join(f"{a} {b[0]:.1e}/{b[1]:.1e}" for a, b in errs.items()))
    bad = {a: b for a, b in errs.items() if not (b[0] <= BAR and b[1] <= BAR_FRO)}
    assert not bad, bad


def _dy(T, d, seed, device="cuda"):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(T, d, generator=g).to(torch.bfloat16).to(device)


def _tbanks(inp):
    routed = {n: inp[n] for n in ("w1", "w3", "w2", "w1_scale", "w3_scale", "w2_scale")}
    rt = pg.moe_mxfp8_transpose_weights(routed)
    st = pg.moe_mxfp8_transpose_weights(inp["shared"]) if inp.get("shared") is not None else None
    return rt, st


def _run(inp, k, dy, replay=False, save_pre=True, ws=None):
    x = inp["x"]
    T, d = x.shape
    E, inter = inp["w_gate"].shape[1], inp["w1"].shape[1]
    ws = ws or pg.BackwardWorkspace(T, d, E, k, inter, pg.MOE_MXFP8)
    fwd = pg.layer_forward(inp, k, ws=ws, replay=replay, save_pre=save_pre)
    bwd = pg.layer_backward(inp, k, fwd, dy, ws, replay=replay, pre=fwd["pre"])
    return fwd, bwd


def _oracle(inp, k, dy, replay=False):
    kw = {}
    if replay:
        kw["ids_in"] = inp["ids_in"].cpu().numpy()
        if inp.get("weights_in") is not None:
            kw["weights_in"] = host(inp["weights_in"])
    return oracle.layer_backward_mxfp8(values(inp["x"], inp["x_scale"]), host(inp["w_gate"]),
                                       host(inp.get("bias")), LazyExperts(inp), shared_of(inp), k,
                                       host(dy), **kw)


def _compare(bwd, ref, E, has_shared, gate):
    errs = {"dx": _errs(host(bwd["dx"]), ref["dx"]),
            "d_weights": _errs(host(bwd["d_weights"]), ref["d_weights"])}
    for n in ("w1", "w3", "w2"):
        got = host(bwd["grads"][n])
        full = np.zeros_like(got)
        for e, v in ref["d" + n].items():
            full[e] = v
        errs["d" + n] = _errs(got, full)
        for e in range(E):          # experts without rows: exactly zero
            if e not in ref["d" + n]:
                assert not got[e].any(), (n, e)
    if has_shared:
        for i, n in enumerate(("w1", "w3", "w2")):
            errs["shared_d" + n] = _errs(host(bwd["shared_grads"][n]), ref["d_shared"][i])
    if gate:
        errs["d_w_gate"] = _errs(host(bwd["d_w_gate"]), ref["d_w_gate"])
        if ref["d_bias"] is not None:
            errs["d_bias"] = _errs(host(bwd["d_bias"]), ref["d_bias"])
    else:
        assert bwd["d_w_gate"] is None
    _check(errs)


def test_transposed_weights_bit_exact():
    wl = synth.Workload("wt", T=4, d=256, inter=128, E=3, k=1, shared=True, dtype="mxfp8", seed=40)
    inp = to_device(synth.make_layer_inputs(wl, device="cpu"))
    say("case MXFP8 requantised weights")
    rt, st = _tbanks(inp)
    for e in range(wl.E):
        w1, w3, w2 = LazyExperts(inp)[e]
        got2 = oracle.mx_dequant(rt["w2t"][e].cpu().numpy(), rt["w2t_scale"][e].cpu().numpy())
        assert np.array_equal(got2, oracle.mx_quantize(w2, 0).T)
        got13 = oracle.mx_dequant(rt["w13t"][e].cpu().numpy(), rt["w13t_scale"][e].cpu().numpy())
        assert np.array_equal(got13[:, :wl.inter], oracle.mx_quantize(w1, 0).T)
        assert np.array_equal(got13[:, wl.inter:], oracle.mx_quantize(w3, 0).T)
    sw1, sw3, sw2 = shared_of(inp)
    assert np.array_equal(oracle.mx_dequant(st["w2t"].cpu().numpy(), st["w2t_scale"].cpu().numpy()),
                          oracle.mx_quantize(sw2, 0).T)


# (name, T, d, I, E, k, shared, bias, routing, seed)
CASES = [
    ("small_learned", 40, 128, 128, 8, 2, True, True, "learned", 41),
    ("ragged_multi_tile", 300, 256, 256, 6, 3, True, False, "learned", 42),
    ("empty_experts", 20, 128, 128, 64, 2, False, True, "learned", 43),
    ("k1_no_shared", 150, 256, 128, 12, 1, False, True, "learned", 44),
    ("replay_gate_weights", 100, 128, 256, 8, 3, True, True, "replay_gate", 45),
    ("replay_caller_weights", 100, 128, 128, 8, 3, True, True, "replay", 46),
    ("ring_forward", 700, 1024, 512, 16, 4, True, True, "learned", 47),   # 256-row forward tiles
]


@pytest.mark.parametrize("name,T,d,I,E,k,shared,bias,routing,seed", CASES, ids=[c[0] for c in CASES])
def test_mxfp8_backward_small_parity(name, T, d, I, E, k, shared, bias, routing, seed):
    wl = synth.Workload(name, T=T, d=d, inter=I, E=E, k=k, shared=shared, bias=bias, dtype="mxfp8",
                        routing="replay" if routing.startswith("replay") else "learned", seed=seed)
    inp = to_device(synth.make_layer_inputs(wl, device="cpu"))
    if routing == "replay_gate":
        inp["weights_in"] = None
    dy = _dy(T, d, seed)
    say(f"case MXFP8 backward {name} T={T} d={d} I={I} E={E} k={k}")
    fwd, bwd = _run(inp, k, dy, replay=routing != "learned")
    ref = _oracle(inp, k, dy, replay=routing != "learned")
    assert np.array_equal(fwd["ids"].cpu().numpy(), ref["ids"])
    _compare(bwd, ref, E, shared, gate=routing != "replay")


def test_mxfp8_backward_recomputed_pre_repeatable_and_token_local():
    wl = synth.Workload("rep", T=260, d=512, inter=512, E=8, k=2, shared=True, bias=True, dtype="mxfp8",
                        seed=48)
    inp = to_device(synth.make_layer_inputs(wl, device="cpu"))
    dy = _dy(wl.T, wl.d, 48)
    say("case MXFP8 backward: saved vs recomputed pre-activations, repeatability, token-local dx")
    _, b0 = _run(inp, wl.k, dy, save_pre=True)
    _, b1 = _run(inp, wl.k, dy, save_pre=False)
    _, b2 = _run(inp, wl.k, dy, save_pre=True)
    for a, b in ((b0, b1), (b0, b2)):
        assert torch.equal(a["dx"], b["dx"]) and torch.equal(a["d_w_gate"], b["d_w_gate"])
        for n in ("w1", "w3", "w2"):
            assert torch.equal(a["grads"][n], b["grads"][n])
            assert torch.equal(a["shared_grads"][n], b["shared_grads"][n])
    for t in (0, 131, 259):
        one = dict(inp, x=inp["x"][t:t + 1].contiguous(), x_scale=inp["x_scale"][t:t + 1].contiguous())
        _, b = _run(one, wl.k, dy[t:t + 1].contiguous())
        assert torch.equal(b["dx"][0], b0["dx"][t])


@pytest.fixture(scope="module")
def full():
    wl = synth.WORKLOADS["mxfp8_t4096"]
    say("drawing an MXFP8 T=4096 layer on the GPU")
    inp = synth.make_layer_inputs(wl, device="cuda")
    dy = torch.randn(wl.T, wl.d, generator=torch.Generator(device="cuda").manual_seed(60),
                     device="cuda").to(torch.bfloat16)
    fwd, bwd = _run(inp, wl.k, dy)
    torch.cuda.synchronize()
    yield wl, inp, dy, fwd, bwd
    del inp, fwd, bwd
    torch.cuda.empty_cache()


def test_mxfp8_backward_fullsize_shared_expert(full):
    wl, inp, dy, fwd, bwd = full
    say("case MXFP8 backward T=4096: the shared expert over every token")
    x = values(inp["x"], inp["x_scale"])
    sh = shared_of(inp)
    a, g, hq, _ = oracle.expert_forward_mxfp8(x, *sh)
    dx, dw1, dw3, dw2, _ = oracle.expert_backward_mxfp8(x, a, g, hq, host(dy), *sh)
    Tk = wl.T * wl.k
    errs = {"dx_rows": _errs(host(bwd["dx_rows"][Tk:]), dx)}
    for n, ref in (("w1", dw1), ("w3", dw3), ("w2", dw2)):
        errs["d" + n] = _errs(host(bwd["shared_grads"][n]), ref)
    _check(errs)


def test_mxfp8_backward_fullsize_routed_expert(full):
    wl, inp, dy, fwd, bwd = full
    off = fwd["offsets"].cpu().numpy()
    e = int(np.argmax(np.diff(off)))
    lo, hi = int(off[e]), int(off[e + 1])
    say(f"case MXFP8 backward T=4096: routed expert {e} ({hi - lo} rows)")
    toks = torch.from_numpy(fwd["perm"].cpu().numpy()[lo:hi] // wl.k).cuda()
    x = values(inp["x"][toks], inp["x_scale"][toks])
    ws = LazyExperts(inp)[e]
    a, g, hq, _ = oracle.expert_forward_mxfp8(x, *ws)
    d_out = host(bwd["d_out"][lo:hi])
    dx, dw1, dw3, dw2, _ = oracle.expert_backward_mxfp8(x, a, g, hq, d_out, *ws)
    errs = {"dx_rows": _errs(host(bwd["dx_rows"][lo:hi]), dx)}
    for n, ref in (("w1", dw1), ("w3", dw3), ("w2", dw2)):
        errs["d" + n] = _errs(host(bwd["grads"][n][e]), ref)
    _check(errs)
