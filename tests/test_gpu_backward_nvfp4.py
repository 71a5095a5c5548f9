"""GPU parity of the MXFP8 backward of NVFP4 layers (NVFP4 forward, MXFP8 backward)
against the oracle's MXFP8 backward of the NVFP4 forward.

The backward GEMMs take x, the weights and h as the NVFP4 forward quantized them,
requantised to MXFP8 along each GEMM's reduction; the oracle does the same with exact
products and sums.  Bars as for the MXFP8 backward: normwise (max |err| / max |ref|)
6e-2, relative Frobenius 1e-2.  Also checked: the weights requantised from NVFP4 are
bit-exact against the oracle's quantiser of the exact NVFP4 values; the backward is
bitwise repeatable; at full size (T = 4096, d = 7168, I = 2048) the shared expert over
every token and the largest routed expert, against the oracle's expert backward.
"""
import numpy as np
import pytest
import torch

import oracle
import parity_gate_gemm_amd as pg
import synth
from _gpu_common import host, say, to_device

pytestmark = pytest.mark.gpu

BAR = 6e-2
BAR_FRO = 1e-2


def _errs(got, ref):
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


def _unpack(packed):
    p = packed.cpu().numpy()
    return np.stack([p & 15, p >> 4], axis=-1).reshape(p.shape[0], -1)


def _triples(b, e):
    """The oracle's (codes, block scales, row scales) of one row-major NVFP4 expert."""
    pick = (lambda t: t[e]) if e is not None else (lambda t: t)
    return tuple((_unpack(pick(b[n])), pick(b[n + "_scale"]).cpu().numpy(), pick(b[n + "_rscale"]).cpu().numpy())
                 for n in ("w1", "w3", "w2"))


class _Experts:
    def __init__(self, inp):
        self.inp = inp

    def __getitem__(self, e):
        return _triples(self.inp, e)


def _shared(inp):
    return _triples(inp["shared"], None) if inp.get("shared") is not None else None


def _run(inp, k, dy, replay=False):
    packed = pg.nvfp4_pack_inputs(inp)
    T, d = inp["x"].shape
    E, inter = inp["w_gate"].shape[1], inp["w1"].shape[1]
    ws = pg.BackwardWorkspace(T, d, E, k, inter, pg.MOE_NVFP4)
    fwd = pg.layer_forward(packed, k, ws=ws, replay=replay, save_pre=True)
    bwd = pg.layer_backward(packed, k, fwd, dy, ws, replay=replay, pre=fwd["pre"])
    return fwd, bwd


def test_nvfp4_transposed_weights_bit_exact():
    wl = synth.Workload("wt", T=4, d=256, inter=128, E=3, k=1, shared=True, dtype="nvfp4", seed=50)
    inp = to_device(synth.make_layer_inputs(wl, device="cpu"))
    say("case NVFP4 weights requantised to MXFP8")
    packed = pg.nvfp4_pack_inputs(inp)
    rt = pg.moe_mxfp8_transpose_weights({n: packed[n] for n in ("w1", "w3", "w2") + pg._BANK_OPT})
    for e in range(wl.E):
        W1, W3, W2 = (oracle.nvfp4_dequant(*t) for t in _triples(inp, e))
        got2 = oracle.mx_dequant(rt["w2t"][e].cpu().numpy(), rt["w2t_scale"][e].cpu().numpy())
        assert np.array_equal(got2, oracle.mx_quantize(W2, 0).T)
        got13 = oracle.mx_dequant(rt["w13t"][e].cpu().numpy(), rt["w13t_scale"][e].cpu().numpy())
        assert np.array_equal(got13[:, :wl.inter], oracle.mx_quantize(W1, 0).T)
        assert np.array_equal(got13[:, wl.inter:], oracle.mx_quantize(W3, 0).T)


# (name, T, d, I, E, k, shared, bias, routing, seed)
CASES = [
    ("small_learned", 40, 256, 128, 8, 2, True, True, "learned", 51),
    ("ragged_multi_tile", 300, 512, 256, 6, 3, True, False, "learned", 52),
    ("k1_no_shared", 150, 256, 128, 12, 1, False, True, "learned", 53),
    ("replay_caller_weights", 100, 256, 256, 8, 3, True, True, "replay", 54),
]


@pytest.mark.parametrize("name,T,d,I,E,k,shared,bias,routing,seed", CASES, ids=[c[0] for c in CASES])
def test_nvfp4_backward_small_parity(name, T, d, I, E, k, shared, bias, routing, seed):
    wl = synth.Workload(name, T=T, d=d, inter=I, E=E, k=k, shared=shared, bias=bias, dtype="nvfp4",
                        routing="replay" if routing == "replay" else "learned", seed=seed)
    inp = to_device(synth.make_layer_inputs(wl, device="cpu"))
    g = torch.Generator().manual_seed(seed)
    dy = torch.randn(T, d, generator=g).to(torch.bfloat16).cuda()
    say(f"case NVFP4-forward MXFP8 backward {name} T={T} d={d} I={I} E={E} k={k}")
    replay = routing == "replay"
    fwd, bwd = _run(inp, k, dy, replay=replay)
    kw = {"ids_in": inp["ids_in"].cpu().numpy(), "weights_in": host(inp["weights_in"])} if replay else {}
    ref = oracle.layer_backward_mxfp8(host(inp["x"]), host(inp["w_gate"]), host(inp.get("bias")), _Experts(inp),
                                      _shared(inp), k, host(dy), forward="nvfp4", **kw)
    assert np.array_equal(fwd["ids"].cpu().numpy(), ref["ids"])
    errs = {"dx": _errs(host(bwd["dx"]), ref["dx"]), "d_weights": _errs(host(bwd["d_weights"]), ref["d_weights"])}
    for n in ("w1", "w3", "w2"):
        got = host(bwd["grads"][n])
        full = np.zeros_like(got)
        for e, v in ref["d" + n].items():
            full[e] = v
        errs["d" + n] = _errs(got, full)
        for e in range(E):
            if e not in ref["d" + n]:
                assert not got[e].any(), (n, e)
    if shared:
        for i, n in enumerate(("w1", "w3", "w2")):
            errs["shared_d" + n] = _errs(host(bwd["shared_grads"][n]), ref["d_shared"][i])
    if not replay:
        errs["d_w_gate"] = _errs(host(bwd["d_w_gate"]), ref["d_w_gate"])
    _check(errs)
    _, again = _run(inp, k, dy, replay=replay)
    assert torch.equal(again["dx"], bwd["dx"])
    for n in ("w1", "w3", "w2"):
        assert torch.equal(again["grads"][n], bwd["grads"][n])


@pytest.fixture(scope="module")
def full():
    wl = synth.WORKLOADS["nvfp4_t4096"]
    say("drawing nvfp4_t4096 inputs on the GPU")
    inp = synth.make_layer_inputs(wl, device="cuda")
    dy = torch.randn(wl.T, wl.d, generator=torch.Generator(device="cuda").manual_seed(70),
                     device="cuda").to(torch.bfloat16)
    fwd, bwd = _run(inp, wl.k, dy)
    torch.cuda.synchronize()
    yield wl, inp, dy, fwd, bwd
    del inp, fwd, bwd
    torch.cuda.empty_cache()


def test_nvfp4_backward_fullsize_shared_expert(full):
    wl, inp, dy, fwd, bwd = full
    say("case NVFP4-forward MXFP8 backward T=4096: the shared expert over every token")
    xq, a, g, hq, _, wv = oracle.expert_forward_nvfp4(host(inp["x"]), *_shared(inp))
    dx, dw1, dw3, dw2, _ = oracle.expert_backward_mxfp8(xq, a, g, hq, host(dy), *wv)
    Tk = wl.T * wl.k
    errs = {"dx_rows": _errs(host(bwd["dx_rows"][Tk:]), dx)}
    for n, ref in (("w1", dw1), ("w3", dw3), ("w2", dw2)):
        errs["d" + n] = _errs(host(bwd["shared_grads"][n]), ref)
    _check(errs)


def test_nvfp4_backward_fullsize_routed_expert(full):
    wl, inp, dy, fwd, bwd = full
    off = fwd["offsets"].cpu().numpy()
    e = int(np.argmax(np.diff(off)))
    lo, hi = int(off[e]), int(off[e + 1])
    say(f"case NVFP4-forward MXFP8 backward T=4096: routed expert {e} ({hi - lo} rows)")
    toks = torch.from_numpy(fwd["perm"].cpu().numpy()[lo:hi] // wl.k).cuda()
    xq, a, g, hq, _, wv = oracle.expert_forward_nvfp4(host(inp["x"][toks]), *_triples(inp, e))
    dx, dw1, dw3, dw2, _ = oracle.expert_backward_mxfp8(xq, a, g, hq, host(bwd["d_out"][lo:hi]), *wv)
    errs = {"dx_rows": _errs(host(bwd["dx_rows"][lo:hi]), dx)}
    for n, ref in (("w1", dw1), ("w3", dw3), ("w2", dw2)):
        errs["d" + n] = _errs(host(bwd["grads"][n][e]), ref)
    _check(errs)
