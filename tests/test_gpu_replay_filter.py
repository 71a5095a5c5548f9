"""GPU parity of router replay with the plausibility filter (moe_route_replay_filtered).

Against the oracle: ids bit-exact, weights within 2e-6 (fp32 weights vs the fp64
oracle), device flag clean.  log_tau = -inf and +inf must reproduce plain replay and
learned routing bit for bit.  Thresholds set to one token's exact logit difference
(kept: the test is >=) and to the next double above it (dropped) sit on the decision
boundary, where the fp64 bound cannot decide and the exact-summation pass must.

Replayed ids are built per row from the oracle's own ranking: the router's set
permuted, the set with columns swapped for the next-ranked experts, the set with one
column swapped for the lowest-ranked expert, and random distinct ids.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parity_gate_gemm_amd as pg
import synth
from _gpu_common import WEIGHT_TOL, host, say, values

pytestmark = pytest.mark.gpu

_DT = {"f32": pg.MOE_F32, "bf16": pg.MOE_BF16, "mxfp8": pg.MOE_MXFP8}


def _gate_inputs(wl, device="cpu"):
    g = synth.make_gate_inputs(wl, device="cpu")
    return {kk: (v.to("cuda") if v is not None else None) for kk, v in g.items()}


def _host_gate(g):
    return values(g["x"], g["x_scale"]), host(g["w_gate"]), host(g["bias"])


def _replay_ids(logits, k, seed):
    """Replayed ids from the oracle's ranking (see the module docstring)."""
    rng = np.random.default_rng(seed)
    T, E = logits.shape
    rank = np.array([sorted(range(E), key=lambda e: (-logits[t, e], e)) for t in range(T)])
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        kind = t % 4
        row = rank[t, :k].copy()
        if kind == 0 or E == k:
            row = rng.permutation(row)
        elif kind == 1:
            m = min(E - k, k, 1 + t % 2)
            cols = rng.choice(k, size=m, replace=False)
            row[cols] = rank[t, k:k + m]
            row = rng.permutation(row)
        elif kind == 2:
            row[rng.integers(k)] = rank[t, E - 1]
        else:
            row = rng.permutation(E)[:k]
        ids[t] = row
    return ids


def _boundary_taus(logits, ids_in, k):
    """(tau on the boundary of a column that is not the router's k-th, next double up)."""
    T = logits.shape[0]
    for t in range(T):
        rk = sorted(range(logits.shape[1]), key=lambda e: (-logits[t, e], e))[k - 1]
        for j in range(k):
            q = int(ids_in[t, j])
            if q != rk:
                lt = float(logits[t, q]) - float(logits[t, rk])
                return [lt, math.nextafter(lt, math.inf)]
    return []


def _run(g, ids_in, lt, ws, k):
    return pg.moe_route_replay_filtered(g["x"], g["w_gate"], g["bias"], ids_in, lt, ws,
                                        x_scale=g["x_scale"])


def _check_against_oracle(g, hg, ids_in_np, lt, ws, k):
    ids_in = torch.from_numpy(ids_in_np).cuda()
    ids, w = _run(g, ids_in, lt, ws, k)
    assert pg.moe_check(ws) == 0
    rid, rw, keep, _ = oracle.route_replay_filtered(*hg, ids_in_np, lt)
    got = ids.cpu().numpy()
    bad = np.nonzero((got != rid).any(axis=1))[0]
    assert bad.size == 0, (lt, bad[:5], got[bad[:5]], rid[bad[:5]])
    err = np.max(np.abs(w.cpu().numpy().astype(np.float64) - rw))
    assert err <= WEIGHT_TOL, (lt, err)
    return ids, w, keep


# (name, T, d, E, k, bias, dtype): unscreened fp64-GEMM gate (fp32; d % 64 != 0),
# screened gate with whole-batch tiles and with the split small-batch gate, k = 1, k = E.
SMALL = [
    ("f32_gemm_gate", 96, 128, 32, 4, True, "f32"),
    ("bf16_d96_gemm_gate", 80, 96, 24, 3, False, "bf16"),
    ("bf16_screened", 300, 256, 64, 8, True, "bf16"),
    ("bf16_split_gate", 64, 1024, 64, 8, True, "bf16"),
    ("mxfp8_screened", 260, 256, 96, 6, True, "mxfp8"),
    ("mxfp8_split_gate", 40, 512, 48, 8, False, "mxfp8"),
    ("bf16_k1", 50, 128, 16, 1, False, "bf16"),
    ("bf16_k_eq_E", 30, 128, 8, 8, True, "bf16"),
]


@pytest.mark.parametrize("name,T,d,E,k,bias,dtype", SMALL, ids=[c[0] for c in SMALL])
def test_filter_small_parity(name, T, d, E, k, bias, dtype):
    wl = synth.Workload(name, T=T, d=d, inter=64, E=E, k=k, bias=bias, dtype=dtype, seed=21)
    g = _gate_inputs(wl)
    hg = _host_gate(g)
    logits = oracle.exact_logits(*hg)
    ids_in_np = _replay_ids(logits, k, seed=5)
    ws = pg.Workspace(T, d, E, k, 64, _DT[dtype])
    taus = [-math.inf, math.log(0.5), -2.0, 0.0, 1.0, math.inf] + _boundary_taus(logits, ids_in_np, k)
    for lt in taus:
        say(f"case filter {name} log_tau {lt!r}")
        _check_against_oracle(g, hg, ids_in_np, lt, ws, k)
    # the limits, bit for bit against the other two entry points
    ids_in = torch.from_numpy(ids_in_np).cuda()
    ids, w = _run(g, ids_in, -math.inf, ws, k)
    w_rep = pg.moe_route_replay(g["x"], g["w_gate"], g["bias"], ids_in, ws, x_scale=g["x_scale"])
    assert torch.equal(ids, ids_in) and torch.equal(w, w_rep)
    ids, w = _run(g, ids_in, math.inf, ws, k)
    lid, lw = pg.moe_route(g["x"], g["w_gate"], g["bias"], k, ws, x_scale=g["x_scale"])
    assert torch.equal(ids, lid) and torch.equal(w, lw)
    assert pg.moe_check(ws) == 0


def test_filter_boundary_many_tokens():
    """Every token sits on its own boundary in turn: one call per token with log_tau
    equal to that token's exact difference; all tokens' ids must match the oracle."""
    wl = synth.Workload("bnd", T=24, d=256, inter=64, E=32, k=4, bias=True, dtype="bf16", seed=8)
    g = _gate_inputs(wl)
    hg = _host_gate(g)
    logits = oracle.exact_logits(*hg)
    ids_in_np = _replay_ids(logits, wl.k, seed=9)
    ws = pg.Workspace(wl.T, wl.d, wl.E, wl.k, 64, pg.MOE_BF16)
    for t in range(0, wl.T, 3):
        taus = _boundary_taus(logits[t:t + 1], ids_in_np[t:t + 1], wl.k)
        for lt in taus:
            say(f"case boundary token {t} log_tau {lt!r}")
            _check_against_oracle(g, hg, ids_in_np, lt, ws, wl.k)


def test_filter_bad_ids_flagged_rows_get_router_choice():
    wl = synth.Workload("badf", T=40, d=128, inter=64, E=16, k=4, bias=False, dtype="bf16", seed=3)
    g = _gate_inputs(wl)
    hg = _host_gate(g)
    logits = oracle.exact_logits(*hg)
    ids_np = _replay_ids(logits, wl.k, seed=1)
    ids_np[3, 2] = 16
    ids_np[7, 1] = ids_np[7, 0]
    ws = pg.Workspace(wl.T, wl.d, wl.E, wl.k, 64, pg.MOE_BF16)
    say("case filter bad ids")
    ids, w = _run(g, torch.from_numpy(ids_np).cuda(), math.log(0.5), ws, wl.k)
    assert pg.moe_check(ws) == 4           # MOE_ERR_BAD_IDS
    got = ids.cpu().numpy()
    router = oracle.topk_ids(logits, wl.k)
    assert np.array_equal(got[[3, 7]], router[[3, 7]])
    good = np.setdiff1d(np.arange(wl.T), [3, 7])
    rid, rw, _, _ = oracle.route_replay_filtered(hg[0][good], hg[1], hg[2], ids_np[good], math.log(0.5))
    assert np.array_equal(got[good], rid)
    assert np.max(np.abs(w.cpu().numpy()[good] - rw)) <= WEIGHT_TOL


def test_filter_empty_batch_and_permutation():
    ws0 = pg.Workspace(0, 128, 16, 2, 64, pg.MOE_BF16)
    x = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    wg = torch.zeros(128, 16, device="cuda")
    ids, w = pg.moe_route_replay_filtered(x, wg, None, torch.empty(0, 2, dtype=torch.int32, device="cuda"),
                                          0.0, ws0)
    assert ids.shape == (0, 2) and w.shape == (0, 2)
    wl = synth.Workload("perm", T=200, d=256, inter=64, E=64, k=8, bias=True, dtype="bf16", seed=4)
    g = _gate_inputs(wl)
    hg = _host_gate(g)
    ids_np = _replay_ids(oracle.exact_logits(*hg), wl.k, seed=2)
    ws = pg.Workspace(wl.T, wl.d, wl.E, wl.k, 64, pg.MOE_BF16)
    ids_in = torch.from_numpy(ids_np).cuda()
    say("case filter permutation")
    a_ids, a_w = _run(g, ids_in, math.log(0.25), ws, wl.k)
    p = torch.randperm(wl.T, generator=torch.Generator().manual_seed(3)).cuda()
    gp = dict(g, x=g["x"][p].contiguous())
    b_ids, b_w = _run(gp, ids_in[p].contiguous(), math.log(0.25), ws, wl.k)
    assert torch.equal(b_ids, a_ids[p]) and torch.equal(b_w, a_w[p])


# ---------------------------------------------------------------------------
# Full workload sizes
# ---------------------------------------------------------------------------
def _inference_like_ids(g, k):
    """Replayed ids as a lower-precision inference engine would pick them: the top k
    of fp32 logits from a plain torch matmul of the decoded activations."""
    x = g["x"]
    T, d = x.shape
    if g["x_scale"] is not None:
        table = torch.tensor(np.asarray(oracle.E4M3_TABLE, dtype=np.float32), device=x.device)
        sc = torch.exp2(g["x_scale"].float() - 127.0).unsqueeze(-1)
        xf = (table[x.long()].view(T, d // 32, 32) * sc).view(T, d)
    else:
        xf = x.float()
    lg = xf @ g["w_gate"]
    if g["bias"] is not None:
        lg = lg + g["bias"]
    return torch.topk(lg, k, dim=1).indices.to(torch.int32).contiguous()


FULL = [("bf16_t4096", synth.WORKLOADS["replay_zipf_t4096"].with_(routing="learned")),
        ("mxfp8_t32768", synth.WORKLOADS["mxfp8_t32768"])]


@pytest.mark.parametrize("name,wl", FULL, ids=[c[0] for c in FULL])
def test_filter_fullsize_sampled(name, wl):
    say(f"drawing {name} gate inputs on the GPU")
    g = synth.make_gate_inputs(wl, device="cuda")
    T, k = wl.T, wl.k
    ws = pg.Workspace(T, wl.d, wl.E, k, wl.inter, _DT[wl.dtype])
    lid, lw = pg.moe_route(g["x"], g["w_gate"], g["bias"], k, ws, x_scale=g["x_scale"])
    router = lid.cpu().numpy()
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    kinds = [("inference", _inference_like_ids(g, k)),
             ("zipf", torch.from_numpy(synth.zipf_replay_ids(T, wl.E, k, 1.2, rng)).cuda())]
    srng = np.random.default_rng(7)
    for kind, ids_in in kinds:
        qin = ids_in.cpu().numpy()
        say(f"case {name} {kind}: rows whose replayed set differs from the router's: "
            f"{int((np.sort(qin, 1) != np.sort(router, 1)).any(1).sum())}")
        for lt in [math.log(0.5), 0.0]:
            say(f"case {name} {kind} log_tau {lt!r}")
            ids, w = _run(g, ids_in, lt, ws, k)
            assert pg.moe_check(ws) == 0
            got = ids.cpu().numpy()
            # every row: distinct ids; a column keeps its replayed id or takes a router id
            srt = np.sort(got, 1)
            assert (np.diff(srt, axis=1) > 0).all() and got.min() >= 0 and got.max() < wl.E
            changed = got != qin
            assert all(set(got[t][changed[t]].tolist()) <= set(router[t].tolist()) for t in range(T))
            acted = np.nonzero(changed.any(1))[0]
            rows = set(srng.choice(acted, size=min(10, acted.size), replace=False).tolist()) if acted.size else set()
            rows |= set(srng.integers(0, T, size=4).tolist()) | {T - 1}
            rows = np.array(sorted(rows))
            tr = torch.from_numpy(rows).cuda()
            hx = values(g["x"][tr], None if g["x_scale"] is None else g["x_scale"][tr])
            rid, rw, _, _ = oracle.route_replay_filtered(hx, host(g["w_gate"]), host(g["bias"]), qin[rows], lt)
            assert np.array_equal(got[rows], rid), rows
            assert np.max(np.abs(w.cpu().numpy()[rows].astype(np.float64) - rw)) <= WEIGHT_TOL
            say(f"  filter acted on {acted.size} rows; oracle rows {rows.tolist()}")
        ids, w = _run(g, ids_in, -math.inf, ws, k)
        w_rep = pg.moe_route_replay(g["x"], g["w_gate"], g["bias"], ids_in, ws, x_scale=g["x_scale"])
        assert torch.equal(ids, ids_in) and torch.equal(w, w_rep)
        ids, w = _run(g, ids_in, math.inf, ws, k)
        assert torch.equal(ids, lid) and torch.equal(w, lw)
        assert pg.moe_check(ws) == 0
    del g, ws
    torch.cuda.empty_cache()
