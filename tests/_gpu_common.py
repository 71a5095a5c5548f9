"""Shared helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import parity_gate_gemm_amd as pg

TOL = {"f32": 2e-2, "bf16": 2e-2, "mxfp8": 6e-2}   # normwise max-abs-rel bar
WEIGHT_TOL = 2e-6                                   # fp32 weights vs fp64 oracle
# Relative Frobenius bars where the arithmetic fixes a much smaller error than the normwise
# bar: bf16 layers round h, the expert outputs and y to bf16 (each an element error of at
# most 2^-9, about 1.1e-3 rms; measured 2.4-3.1e-3 together); the fp32 layer accumulates
# in fp32 over d + I terms (measured 2-5e-7).  MXFP8 layers: FROB_MX_HQ below.
FROB = {"f32": 1e-5, "bf16": 6e-3}
# MXFP8 layers against the oracle that requantises h per row as the library does
# (oracle.layer_mxfp8): what is left is the bf16 rounding of the expert outputs and of y
# (relative Frobenius error about 2.5e-3) and the rare E4M3 code, or block scale, that a
# last-bit difference of h moves across a rounding boundary.  Such a flip can show in
# the largest elements of a row (normwise up to 4.6e-2 measured), so the normwise bar
# stays the MXFP8 one and the relative Frobenius error, which isolated flips barely move,
# must stay below 6e-3 (against the exact h it is about 2.7e-2).
FROB_MX_HQ = 6e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    """Stored values of a device/host tensor as float64 numpy (exact)."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64) if t.dtype != torch.int32 else t.cpu().numpy()


def values(t, scale=None):
    """Exact float64 values of a stored tensor; MXFP8 codes are dequantised by the
    oracle's own decoder."""
    if scale is None:
        return host(t)
    return oracle.mx_dequant(t.cpu().numpy(), scale.cpu().numpy())


class LazyExperts:
    """experts[e] -> (w1, w3, w2) float64 numpy, fetched from device tensors on demand."""

    def __init__(self, inp):
        self.inp = inp

    def __getitem__(self, e):
        sc = lambda n: None if self.inp.get(n + "_scale") is None else self.inp[n + "_scale"][e]  # noqa: E731
        return tuple(values(self.inp[n][e], sc(n)) for n in ("w1", "w3", "w2"))


def shared_of(inp):
    sh = inp.get("shared")
    if sh is None:
        return None
    return tuple(values(sh[n], sh.get(n + "_scale")) for n in ("w1", "w3", "w2"))


def to_device(inp, device="cuda"):
    out = {}
    for kk, v in inp.items():
        if isinstance(v, torch.Tensor):
            out[kk] = v.to(device)
        elif isinstance(v, dict):
            out[kk] = {a: (b.to(device) if isinstance(b, torch.Tensor) else b) for a, b in v.items()}
        else:
            out[kk] = v
    return out


def oracle_for_rows(inp, rows, k, replay=False, layer=oracle.layer):
    """Oracle layer on a subset of token rows (routing and FFN are row-local);
    ``layer=oracle.layer_mxfp8`` for the MXFP8 layer with h requantised."""
    xs = inp.get("x_scale")
    x = values(inp["x"][rows], None if xs is None else xs[rows])
    kw = {}
    if replay:
        kw["ids_in"] = inp["ids_in"].cpu().numpy()[rows]
        if inp.get("weights_in") is not None:
            kw["weights_in"] = host(inp["weights_in"])[rows]
    return layer(x, host(inp["w_gate"]), host(inp.get("bias")), LazyExperts(inp),
                 shared_of(inp), k, **kw)


def compare_rows(res_gpu, ref, rows, dtype, replay=False):
    """ids bit-exact, weights within WEIGHT_TOL, y normwise within the dtype's bar (and
    within its relative Frobenius bar, where it has one)."""
    ids = res_gpu["ids"].cpu().numpy()[rows]
    assert np.array_equal(ids, ref["ids"]), (ids, ref["ids"])
    w = res_gpu["weights"].cpu().numpy()[rows].astype(np.float64)
    assert np.max(np.abs(w - ref["weights"])) <= WEIGHT_TOL, np.max(np.abs(w - ref["weights"]))
    y = host(res_gpu["y"])[rows]
    err = oracle.normwise_rel_err(y, ref["y"])
    fr = float(np.linalg.norm(y - ref["y"]) / max(np.linalg.norm(ref["y"]), 1e-300))
    say(f"  normwise err {err:.3e} (bar {TOL[dtype]}), relative Frobenius {fr:.3e} "
        f"(bar {FROB.get(dtype, '-')})")
    assert err <= TOL[dtype], err
    if dtype in FROB:
        assert fr <= FROB[dtype], fr
    return err


def compare_rows_hq(res_gpu, ref_mx, rows):
    """An MXFP8 layer's y against ``oracle.layer_mxfp8`` on the same rows: normwise
    within the MXFP8 bar and relative Frobenius error within FROB_MX_HQ."""
    y = host(res_gpu["y"])[rows]
    nw = oracle.normwise_rel_err(y, ref_mx["y"])
    fr = float(np.linalg.norm(y - ref_mx["y"]) / np.linalg.norm(ref_mx["y"]))
    say(f"  against the requantised h: normwise {nw:.3e} (bar {TOL['mxfp8']}), "
        f"Frobenius {fr:.3e} (bar {FROB_MX_HQ})")
    assert nw <= TOL["mxfp8"], nw
    assert fr <= FROB_MX_HQ, fr
    return fr


def check_routing_every_token(inp, res, k, E):
    """Every token's ids bit-exact against the oracle's certified routing (the ids of
    ``oracle.route``), every weight within WEIGHT_TOL, and offsets / perm / row_of equal
    to ``oracle.dispatch`` of the oracle's ids."""
    x = values(inp["x"], inp.get("x_scale"))
    ids, w, n_exact = oracle.route_certified(x, host(inp["w_gate"]), host(inp.get("bias")), k)
    del x
    gids = res["ids"].cpu().numpy()
    T = ids.shape[0]
    bad = np.nonzero((gids != ids).any(axis=1))[0]
    say(f"  ids exact on {T - len(bad)}/{T} tokens ({n_exact} decided by exact sums in the oracle)")
    assert len(bad) == 0, bad[:10]
    gw = res["weights"].cpu().numpy().astype(np.float64)
    werr = float(np.max(np.abs(gw - w))) if T else 0.0
    say(f"  weights max abs err {werr:.2e} over {T} tokens")
    assert werr <= WEIGHT_TOL
    off, perm, row_of = oracle.dispatch(ids, E)
    assert np.array_equal(res["offsets"].cpu().numpy(), off)
    assert np.array_equal(res["perm"].cpu().numpy(), perm)
    assert np.array_equal(res["row_of"].cpu().numpy(), row_of)
    say(f"  offsets, perm and row_of exact on {T * k} pairs")
    return ids


def sample_rows(ids, offsets, perm, k, tile, shared, n, seed):
    """About n token rows that cover the grouped GEMM's edge cases: the first and last
    token of the largest segment and the tokens on its first row-tile boundaries, the
    last token of the largest segment with a ragged (partial) last tile, tokens on the
    shared expert's tile boundaries, the first and last token, then random tokens."""
    ids = np.asarray(ids)
    off = np.asarray(offsets).astype(np.int64)
    perm = np.asarray(perm).astype(np.int64)
    T = ids.shape[0]
    seg = np.diff(off)
    rows = {0, T - 1}
    e_big = int(np.argmax(seg))
    toks = perm[off[e_big]:off[e_big + 1]] // k
    rows |= {int(toks[0]), int(toks[-1])}
    for b in range(tile, min(len(toks), 3 * tile + 1), tile):
        rows |= {int(toks[b - 1]), int(toks[b])}
    ragged = [e for e in range(len(seg)) if seg[e] % tile]
    if ragged:
        e_r = max(ragged, key=lambda e: seg[e])
        rows.add(int(perm[off[e_r + 1] - 1] // k))
    if shared:
        for b in range(tile, min(T, 3 * tile + 1), tile):
            rows |= {b - 1, b}
        rows |= {T // 2, (T // tile) * tile - 1}
    rng = np.random.default_rng(seed)
    while len(rows) < min(n, T):
        rows.add(int(rng.integers(0, T)))
    rows = {r for r in rows if 0 <= r < T}
    return np.array(sorted(rows))


def check_dispatch_properties(ids_gpu, offsets, perm, row_of, E):
    """Properties that pin the counting sort at any size (computed on the host)."""
    ids = ids_gpu.cpu().numpy().astype(np.int64)
    off = offsets.cpu().numpy().astype(np.int64)
    pm = perm.cpu().numpy().astype(np.int64)
    ro = row_of.cpu().numpy().astype(np.int64)
    T, k = ids.shape
    assert off[0] == 0 and off[E] == T * k
    assert np.array_equal(np.diff(off), np.bincount(ids.ravel(), minlength=E))
    assert np.array_equal(np.sort(pm), np.arange(T * k))
    assert np.array_equal(pm[ro], np.arange(T * k))
    seg_e = np.repeat(np.arange(E), np.diff(off))
    assert np.array_equal(ids.ravel()[pm], seg_e)
    key = seg_e * (T * k) + pm             # (expert, token, slot) ascending
    assert np.all(np.diff(key) > 0)


def run_layer(inp, k, replay=False, ws=None):
    return pg.layer_forward(inp, k, ws=ws, replay=replay)
