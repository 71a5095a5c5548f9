"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle function to exact rational arithmetic, a closed form,
brute force, an independent formulation, or a hand-derived fixture, chosen so a
dropped term, a wrong sign or index, or a transposed operand fails at least one.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(a):
    return np.asarray(a, dtype=np.float32)


def _bf16_values(rng, shape, scale=1.0):
    """Random values exactly representable in bf16 (top 16 bits of an fp32)."""
    v = _f32(rng.standard_normal(shape) * scale)
    u = v.view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


# ---------------------------------------------------------------------------
# logits
# ---------------------------------------------------------------------------
def _rational_logits(x, w, b):
    T, d = x.shape
    E = w.shape[1]
    out = np.empty((T, E))
    for t in range(T):
        for e in range(E):
            s = sum(Fraction(float(x[t, i])) * Fraction(float(w[i, e])) for i in range(d))
            if b is not None:
                s += Fraction(float(b[e]))
            out[t, e] = float(s)       # Fraction -> float rounds correctly
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_logits_equal_rational_arithmetic(seed):
    rng = np.random.default_rng(seed)
    T, d, E = 4, 9, 7
    x = _bf16_values(rng, (T, d))
    w = _f32(rng.standard_normal((d, E)) / 3)
    b = _f32(rng.standard_normal(E))
    # add cancellation-heavy columns: big +/- pairs around small terms
    w[:, 0] = _f32([2.0 ** 60, 1.0, -(2.0 ** 60), 3.0, -3.0, 2.0 ** -30, 1e20, -1e20, 0.5])
    x[:, :] = np.where(np.arange(d)[None, :] < 9, x, x)
    x[0] = 1.0
    got = oracle.exact_logits(x, w, b)
    want = _rational_logits(x, w, b)
    assert np.array_equal(got, want)


def test_exact_logits_beat_naive_summation():
    # (2^60 + 1) - 2^60 is 0 left to right in float64 but exactly 1.
    x = _f32([[1.0, 1.0, 1.0]])
    w = _f32([[2.0 ** 60], [1.0], [-(2.0 ** 60)]])
    assert oracle.exact_logits(x, w)[0, 0] == 1.0
    assert (np.float64(2.0 ** 60) + 1.0) - 2.0 ** 60 == 0.0


def test_unit_vector_gives_gate_row():
    rng = np.random.default_rng(3)
    d, E = 16, 12
    w = _f32(rng.standard_normal((d, E)))
    b = _f32(rng.standard_normal(E))
    for i in (0, 5, d - 1):
        x = np.zeros((1, d), np.float32)
        x[0, i] = 1.0
        assert np.array_equal(oracle.exact_logits(x, w, b)[0], w[i].astype(np.float64) + b)
        assert np.array_equal(oracle.exact_logits(x, w)[0], w[i].astype(np.float64))


def test_zero_input_routes_to_lowest_indices_with_equal_weights():
    d, E, k = 8, 384, 8
    rng = np.random.default_rng(4)
    w = _f32(rng.standard_normal((d, E)))
    ids, wts, logits = oracle.route(np.zeros((3, d), np.float32), w, None, k)
    assert np.all(logits == 0)
    assert np.array_equal(ids, np.tile(np.arange(k), (3, 1)))
    assert np.all(wts == 1.0 / k)


# ---------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------
def _brute_topk(row, k):
    """Rank of e = number of experts that beat it (larger, or equal with lower index)."""
    E = len(row)
    ids = [None] * k
    for e in range(E):
        beaten = sum(1 for j in range(E) if row[j] > row[e] or (row[j] == row[e] and j < e))
        if beaten < k:
            ids[beaten] = e
    return ids


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(10 + seed)
    E = int(rng.integers(3, 11))
    k = int(rng.integers(1, E + 1))
    # few distinct values -> many exact ties
    logits = rng.integers(-3, 4, size=(20, E)).astype(np.float64) / 4
    ids = oracle.topk_ids(logits, k)
    for t in range(20):
        assert list(ids[t]) == _brute_topk(list(logits[t]), k)


def test_topk_set_maximises_sum_when_distinct():
    rng = np.random.default_rng(7)
    E, k = 10, 3
    for _ in range(10):
        row = rng.standard_normal(E)
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(row[list(s)]))
        got = oracle.topk_ids(row[None, :], k)[0]
        assert sorted(got) == sorted(best)
        assert all(row[got[i]] > row[got[i + 1]] for i in range(k - 1))


def test_duplicate_gate_columns_tie_to_lower_index():
    rng = np.random.default_rng(8)
    d, E = 32, 12
    w = _f32(rng.standard_normal((d, E)))
    w[:, 9] = w[:, 2]              # experts 2 and 9 always tie exactly
    x = _bf16_values(rng, (50, d))
    ids, _, logits = oracle.route(x, w, None, 6)
    for t in range(50):
        row = list(ids[t])
        if 2 in row and 9 in row:
            assert row.index(2) < row.index(9)
        if 9 in row:
            assert 2 in row
        assert logits[t, 2] == logits[t, 9]


# ---------------------------------------------------------------------------
# certified routing (the fast form of route for large batches)
# ---------------------------------------------------------------------------
def _mx_values(rng, shape):
    """Random exact MXFP8 values: E4M3 codes times one power of two per 32-block."""
    codes = rng.integers(0, 256, size=shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0             # no NaN codes
    scales = rng.integers(120, 125, size=shape[:-1] + (shape[-1] // 32,)).astype(np.uint8)
    return oracle.mx_dequant(codes, scales)


@pytest.mark.parametrize("kind", ["bf16", "f32", "mxfp8"])
def test_route_certified_equals_route_on_random_inputs(kind):
    rng = np.random.default_rng({"bf16": 40, "f32": 41, "mxfp8": 42}[kind])
    T, d, E, k = 48, 256, 40, 8
    x = {"bf16": lambda: _bf16_values(rng, (T, d)),
         "f32": lambda: _f32(rng.standard_normal((T, d))),
         "mxfp8": lambda: _mx_values(rng, (T, d))}[kind]()
    w = _f32(rng.standard_normal((d, E)) / 16)
    b = _f32(rng.standard_normal(E) * 0.7) if kind != "f32" else None
    ids, wts, n_exact = oracle.route_certified(x, w, b, k)
    ids0, wts0, _ = oracle.route(x, w, b, k)
    assert np.array_equal(ids, ids0)
    assert np.max(np.abs(wts - wts0)) <= 1e-12
    assert n_exact < T


def test_route_certified_ties_and_near_ties():
    """Exact ties (a duplicated gate column), all-equal logits (x = 0) and near ties
    built so that a left-to-right fp64 sum orders two experts the wrong way: column a
    sums 1 + 64 * 2^-53 = 1 + 2^-47 exactly, which such a sum rounds to 1; column b is
    1 + 31 * 2^-52, just below a.  Every token must get route()'s ids."""
    rng = np.random.default_rng(43)
    d, E, k = 72, 12, 4
    w = _f32(rng.standard_normal((d, E)) / 8)
    w[:, 7] = w[:, 3]                                  # experts 3 and 7 tie exactly
    x = _bf16_values(rng, (30, d))
    x[5] = 0.0                                         # every logit 0: ids 0..k-1
    near = np.zeros((4, d), np.float32)
    near[:, 0] = 1.0
    near[:, 1:65] = 2.0 ** -53
    x = np.concatenate([x, near])
    w[:, 10] = 0.0
    w[:65, 10] = 1.0                                   # column a: 1 + 2^-47 on the near rows
    w = w.astype(np.float64)                           # the near-tie weights need fp64
    w[:, 11] = 0.0
    w[0, 11] = 1.0 + 31 * 2.0 ** -52                   # column b
    w[:, 9] = 0.0
    w[0, 9] = 1.0 + 2.0 ** -52                         # a third, lower near-tie column
    ids, wts, n_exact = oracle.route_certified(x, w, None, k)
    ids0, wts0, logits0 = oracle.route(x, w, None, k)
    assert np.array_equal(ids, ids0)
    assert np.max(np.abs(wts - wts0)) <= 1e-12
    assert list(ids[5]) == [0, 1, 2, 3]
    for t in range(30, 34):
        assert list(ids[t][:3]) == [10, 11, 9]         # exact order a > b > third
        assert logits0[t, 10] > logits0[t, 11] > logits0[t, 9]
    for t in range(30):
        row = list(ids[t])
        if 7 in row:
            assert 3 in row and row.index(3) < row.index(7)
    assert n_exact >= 5


# ---------------------------------------------------------------------------
# gate weights
# ---------------------------------------------------------------------------
def test_weights_closed_forms():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((30, 20)) * 3
    # k = 1 -> weight exactly 1
    ids1 = oracle.topk_ids(logits, 1)
    assert np.all(oracle.softmax_pick_renormalise(logits, ids1) == 1.0)
    # k = 2 -> (sigmoid(l0 - l1), sigmoid(l1 - l0))
    ids2 = oracle.topk_ids(logits, 2)
    w2 = oracle.softmax_pick_renormalise(logits, ids2)
    for t in range(30):
        l0, l1 = logits[t, ids2[t, 0]], logits[t, ids2[t, 1]]
        assert abs(w2[t, 0] - 1 / (1 + math.exp(l1 - l0))) < 1e-15
        assert abs(w2[t, 1] - 1 / (1 + math.exp(l0 - l1))) < 1e-15
    # equal logits -> 1/k
    eq = np.zeros((2, 16))
    assert np.allclose(oracle.softmax_pick_renormalise(eq, oracle.topk_ids(eq, 8)), 1 / 8, rtol=0, atol=1e-16)


def test_full_softmax_equals_restricted_form_and_sums_to_one():
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((40, 384)) * 2
    k = 8
    ids = oracle.topk_ids(logits, k)
    w = oracle.softmax_pick_renormalise(logits, ids)
    for t in range(40):
        sel = logits[t, ids[t]]
        ex = [math.exp(v - sel[0]) for v in sel]
        s = math.fsum(ex)
        assert np.allclose(w[t], [v / s for v in ex], rtol=0, atol=1e-15)
        assert abs(math.fsum(w[t]) - 1.0) < 1e-15
        assert all(w[t, r] >= w[t, r + 1] for r in range(k - 1))


# ---------------------------------------------------------------------------
# the parity metric
# ---------------------------------------------------------------------------
def test_normwise_rel_err_hand_values():
    # max |y - y_ref| / max |y_ref| over the whole array, the reference in the
    # denominator: 8 / 2 = 4.  Swapped arguments would give 8 / 8 = 1.
    assert oracle.normwise_rel_err([[2.0, 8.0]], [[2.0, 0.0]]) == 4.0
    assert oracle.normwise_rel_err([[2.0, 0.0]], [[2.0, 8.0]]) == 1.0
    # one max over all rows, not per row: row 0's error 1 over the global max 10
    # is 0.1; a per-row maximum would give 1 / 1 = 1 for row 0.
    y_ref = [[1.0, 0.0], [10.0, 0.0]]
    y = [[2.0, 0.0], [10.0, 0.5]]
    assert oracle.normwise_rel_err(y, y_ref) == 0.1
    # sign of the difference does not matter; equal arrays give 0
    assert oracle.normwise_rel_err([[-3.0]], [[1.0]]) == 4.0
    assert oracle.normwise_rel_err(y_ref, y_ref) == 0.0
    # an all-zero reference: the absolute maximum of y (0 when y is zero too)
    assert oracle.normwise_rel_err([[0.0, -0.25]], [[0.0, 0.0]]) == 0.25
    assert oracle.normwise_rel_err([[0.0]], [[0.0]]) == 0.0


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------
def test_dispatch_golden():
    g = json.load(open(os.path.join(GOLDEN, "dispatch_hand_sorted.json")))
    off, perm, row_of = oracle.dispatch(np.array(g["ids"]), g["E"])
    assert off.tolist() == g["offsets"]
    assert perm.tolist() == g["perm"]
    assert row_of.tolist() == g["row_of"]


@pytest.mark.parametrize("seed", range(4))
def test_dispatch_brute_force_and_invariants(seed):
    rng = np.random.default_rng(20 + seed)
    T, E, k = int(rng.integers(1, 40)), int(rng.integers(1, 30)), 0
    k = int(rng.integers(1, min(E, 6) + 1))
    p = 1.0 / np.arange(1, E + 1) ** 1.5
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    off, perm, row_of = oracle.dispatch(ids, E)
    # brute force: walk experts, then tokens, then slots
    bf = [t * k + r for e in range(E) for t in range(T) for r in range(k) if ids[t, r] == e]
    assert perm.tolist() == bf
    assert off[0] == 0 and off[E] == T * k
    assert np.all(np.diff(off) >= 0)
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(ids.ravel()[seg] == e)
        assert np.all(np.diff(seg // k) > 0)          # tokens strictly ascending
    assert np.array_equal(np.bincount(perm // k, minlength=T), np.full(T, k))
    assert np.array_equal(perm[row_of], np.arange(T * k))
    assert np.array_equal(row_of[perm], np.arange(T * k))


# ---------------------------------------------------------------------------
# expert FFN
# ---------------------------------------------------------------------------
def test_ffn_scalar_closed_form():
    # d = I = 1: x=2, W1=0.5, W3=3, W2=-1.5 -> a=1, g=6, out = -1.5 * 6 * silu(1)
    out = oracle.expert_ffn([[2.0]], [[0.5]], [[3.0]], [[-1.5]])
    assert abs(out[0, 0] - (-9.0 / (1 + math.exp(-1)))) < 1e-15
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15


def test_ffn_zero_cases():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((5, 6))
    w1, w3, w2 = rng.standard_normal((4, 6)), rng.standard_normal((4, 6)), rng.standard_normal((6, 4))
    assert np.all(oracle.expert_ffn(x, np.zeros_like(w1), w3, w2) == 0)
    assert np.all(oracle.expert_ffn(np.zeros_like(x), w1, w3, w2) == 0)


def test_ffn_matches_elementwise_loops_and_layout():
    rng = np.random.default_rng(13)
    n, d, I = 3, 4, 5
    x = rng.standard_normal((n, d))
    w1, w3, w2 = rng.standard_normal((I, d)), rng.standard_normal((I, d)), rng.standard_normal((d, I))
    got = oracle.expert_ffn(x, w1, w3, w2)
    for t in range(n):
        h = []
        for j in range(I):
            a = math.fsum(x[t, i] * w1[j, i] for i in range(d))
            g = math.fsum(x[t, i] * w3[j, i] for i in range(d))
            h.append(a / (1 + math.exp(-a)) * g)
        for c in range(d):
            want = math.fsum(h[j] * w2[c, j] for j in range(I))
            assert abs(got[t, c] - want) < 1e-12
    # swapping W1 and W3 changes the result (silu applies to the W1 branch only)
    assert not np.allclose(oracle.expert_ffn(x, w3, w1, w2), got)


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------
def test_layer_golden_closed_form():
    g = json.load(open(os.path.join(GOLDEN, "tiny_layer_closed_form.json")))
    ev = lambda s: eval(s, {"exp": math.exp, "__builtins__": {}})  # noqa: E731 (fixture expressions)
    experts = [(np.array(g["w1"][e]), np.array(g["w3"][e]), np.array(g["w2"][e])) for e in range(4)]
    res = oracle.layer(np.array(g["x"]), np.array(g["w_gate"]), None, experts, None, g["k"])
    assert res["ids"].tolist() == g["expected_ids"]
    want_w = np.array([[ev(s) for s in row] for row in g["expected_weights_expr"]])
    want_y = np.array([[ev(s) for s in row] for row in g["expected_y_expr"]])
    assert np.allclose(res["weights"], want_w, rtol=0, atol=1e-15)
    assert np.allclose(res["y"], want_y, rtol=0, atol=1e-15)


def _small_layer(seed, T=10, d=8, I=4, E=16, k=4, shared=True, bias=False):
    rng = np.random.default_rng(seed)
    x = _bf16_values(rng, (T, d))
    wg = _f32(rng.standard_normal((d, E)) / math.sqrt(d))
    b = _f32(rng.standard_normal(E)) if bias else None
    experts = [(rng.standard_normal((I, d)) / math.sqrt(d), rng.standard_normal((I, d)) / math.sqrt(d),
                rng.standard_normal((d, I)) / math.sqrt(I)) for _ in range(E)]
    sh = (rng.standard_normal((I, d)), rng.standard_normal((I, d)), rng.standard_normal((d, I))) if shared else None
    return x, wg, b, experts, sh, k


@pytest.mark.parametrize("seed,shared,bias", [(0, True, False), (1, False, True), (2, True, True)])
def test_layer_dispatched_equals_dense(seed, shared, bias):
    x, wg, b, experts, sh, k = _small_layer(seed, shared=shared, bias=bias)
    y = oracle.layer(x, wg, b, experts, sh, k)["y"]
    yd = oracle.layer_dense(x, wg, b, experts, sh, k)
    assert np.max(np.abs(y - yd)) <= 1e-12 * max(1.0, np.max(np.abs(yd)))


def test_layer_token_permutation_permutes_output():
    x, wg, b, experts, sh, k = _small_layer(3, T=12)
    y = oracle.layer(x, wg, b, experts, sh, k)["y"]
    p = np.random.default_rng(5).permutation(12)
    yp = oracle.layer(x[p], wg, b, experts, sh, k)["y"]
    assert np.max(np.abs(yp - y[p])) <= 1e-12


def test_replay_own_ids_equals_learned():
    x, wg, b, experts, sh, k = _small_layer(4, bias=True)
    learned = oracle.layer(x, wg, b, experts, sh, k)
    rep = oracle.layer(x, wg, b, experts, sh, k, ids_in=learned["ids"])
    assert np.array_equal(rep["y"], learned["y"])
    assert np.array_equal(rep["weights"], learned["weights"])
    rep2 = oracle.layer(x, wg, b, experts, sh, k, ids_in=learned["ids"], weights_in=learned["weights"])
    assert np.array_equal(rep2["y"], learned["y"])


def test_replay_weights_used_verbatim_and_column_order_kept():
    x, wg, b, experts, sh, k = _small_layer(5)
    ids = np.array([[3, 1, 7, 0]] * x.shape[0])
    wts = np.tile([0.1, 0.2, 0.3, 0.5], (x.shape[0], 1))   # sums to 1.1: not renormalised
    res = oracle.layer(x, wg, b, experts, sh, k, ids_in=ids, weights_in=wts)
    assert np.array_equal(res["weights"], wts)
    # reversing the column order of (ids, weights) leaves y unchanged in exact terms
    res2 = oracle.layer(x, wg, b, experts, sh, k, ids_in=ids[:, ::-1], weights_in=wts[:, ::-1])
    assert np.max(np.abs(res2["y"] - res["y"])) < 1e-12
    # replay weights from the router at the given ids (no weights passed)
    res3 = oracle.layer(x, wg, b, experts, sh, k, ids_in=ids)
    lg = oracle.exact_logits(x, wg, b)
    for t in range(x.shape[0]):
        ex = np.exp(lg[t, ids[t]] - lg[t, ids[t]].max())
        assert np.allclose(res3["weights"][t], ex / ex.sum(), rtol=0, atol=1e-15)


def test_replay_rejects_bad_ids():
    x, wg, b, experts, sh, k = _small_layer(6)
    T = x.shape[0]
    with pytest.raises(ValueError):
        oracle.route_replay(x, wg, b, np.full((T, k), 16))
    with pytest.raises(ValueError):
        oracle.route_replay(x, wg, b, np.full((T, k), -1))
    bad = np.tile(np.arange(k), (T, 1))
    bad[3, 1] = bad[3, 0]
    with pytest.raises(ValueError):
        oracle.route_replay(x, wg, b, bad)


# ---------------------------------------------------------------------------
# Replay plausibility filter
# ---------------------------------------------------------------------------
def _filter_inputs(seed, T=24, d=32, E=16, k=4, bias=True):
    rng = np.random.default_rng(seed)
    x = _bf16_values(rng, (T, d))
    wg = _f32(rng.standard_normal((d, E)) * 0.2)
    b = _f32(rng.standard_normal(E) * 0.1) if bias else None
    ids_in = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    return x, wg, b, ids_in


def test_replay_filter_golden():
    g = json.load(open(os.path.join(GOLDEN, "replay_filter_hand.json")))
    x = np.asarray(g["x"], dtype=np.float32)
    wg = np.asarray(g["w_gate_rows"], dtype=np.float32)
    for c in g["cases"]:
        ids, w, keep, _ = oracle.route_replay_filtered(x, wg, None, np.asarray(g["ids_in"]), c["log_tau"])
        assert ids.tolist() == c["ids"]
        assert keep.tolist() == c["keep"]
        assert np.allclose(w, np.asarray(c["weights"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", [0, 1])
def test_replay_filter_limits_are_replay_and_learned(seed):
    x, wg, b, ids_in = _filter_inputs(seed)
    k = ids_in.shape[1]
    ids, w, keep, _ = oracle.route_replay_filtered(x, wg, b, ids_in, -math.inf)
    rid, rw, _ = oracle.route_replay(x, wg, b, ids_in)
    assert keep.all() and np.array_equal(ids, rid) and np.array_equal(w, rw)
    ids, w, keep, _ = oracle.route_replay_filtered(x, wg, b, ids_in, math.inf)
    lid, lw, _ = oracle.route(x, wg, b, k)
    assert not keep.any() and np.array_equal(ids, lid) and np.array_equal(w, lw)


@pytest.mark.parametrize("seed", [2, 3])
def test_replay_filter_matches_probability_form(seed):
    """Independent formulation: probabilities from a plain softmax, p_e >= tau p_(k),
    router order from sorting the probabilities, refill by set difference.  Taus are
    taken away from every probability ratio, so the two forms must agree."""
    x, wg, b, ids_in = _filter_inputs(seed, T=40)
    T, k = ids_in.shape
    lg = np.asarray(x, np.float64) @ np.asarray(wg, np.float64) + np.asarray(b, np.float64)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")
    ratios = np.sort(np.concatenate([p[t, ids_in[t]] / p[t, order[t, k - 1]] for t in range(T)]))
    gaps = np.argsort(np.diff(ratios))[::-1][:6]   # taus in the six widest gaps between ratios
    taus = [0.5 * (ratios[i] + ratios[i + 1]) for i in gaps]
    for tau in taus:
        ids, _, keep, _ = oracle.route_replay_filtered(x, wg, b, ids_in, math.log(tau))
        for t in range(T):
            pk = p[t, order[t, k - 1]]
            kp = [p[t, e] >= tau * pk for e in ids_in[t]]
            assert keep[t].tolist() == kp
            kept = [e for e, z in zip(ids_in[t], kp) if z]
            fill = iter([e for e in order[t, :k] if e not in kept])
            assert ids[t].tolist() == [e if z else next(fill) for e, z in zip(ids_in[t], kp)]


@pytest.mark.parametrize("seed", [4, 5])
def test_replay_filter_tau_one_gives_router_set(seed):
    """tau = 1: a replayed expert stays iff it is at least as likely as the router's
    k-th choice, so (no ties) the final set is the router's set."""
    x, wg, b, ids_in = _filter_inputs(seed)
    k = ids_in.shape[1]
    lid, _, _ = oracle.route(x, wg, b, k)
    ids_in = ids_in.copy()
    ids_in[::3] = lid[::3, ::-1]   # some rows replay the router's own set, reversed
    ids, _, keep, _ = oracle.route_replay_filtered(x, wg, b, ids_in, 0.0)
    for t in range(ids.shape[0]):
        assert set(ids[t].tolist()) == set(lid[t].tolist())
        assert keep[t].tolist() == [int(e) in set(lid[t].tolist()) for e in ids_in[t]]
    assert np.array_equal(ids[::3], ids_in[::3])


def test_replay_filter_monotone_in_tau_and_valid():
    x, wg, b, ids_in = _filter_inputs(6, T=32, E=12, k=5)
    T, k = ids_in.shape
    lid, _, _ = oracle.route(x, wg, b, k)
    prev = None
    for lt in [-math.inf, -8.0, -3.0, -1.5, -0.7, -0.2, 0.0, 0.5, math.inf]:
        ids, w, keep, _ = oracle.route_replay_filtered(x, wg, b, ids_in, lt)
        if prev is not None:
            assert not (keep & ~prev).any()   # raising tau never keeps more
        prev = keep
        assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        for t in range(T):
            assert len(set(ids[t].tolist())) == k
            assert np.array_equal(ids[t][keep[t]], ids_in[t][keep[t]])
            assert set(ids[t][~keep[t]].tolist()) <= set(lid[t].tolist())


def test_replay_filter_rejects_bad_ids_and_nan_threshold():
    x, wg, b, ids_in = _filter_inputs(7, T=4)
    bad = ids_in.copy()
    bad[1, 0] = wg.shape[1]
    with pytest.raises(ValueError):
        oracle.route_replay_filtered(x, wg, b, bad, 0.0)
    bad = ids_in.copy()
    bad[2, 1] = bad[2, 0]
    with pytest.raises(ValueError):
        oracle.route_replay_filtered(x, wg, b, bad, 0.0)
    with pytest.raises(ValueError):
        oracle.route_replay_filtered(x, wg, b, ids_in, math.nan)


# ---------------------------------------------------------------------------
# MXFP8 decoding
# ---------------------------------------------------------------------------
def test_e4m3_table_hand_values():
    # OCP MX v1.0 FP8 E4M3: bias 7, subnormal step 2^-9, max 448, S.1111.111 NaN
    assert oracle.e4m3_value(0x00) == 0.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x3C) == 1.5
    assert oracle.e4m3_value(0x7E) == 448.0
    assert math.isnan(oracle.e4m3_value(0x7F))
    assert oracle.e4m3_value(0xFE) == -448.0
    assert oracle.e4m3_value(0xB8) == -1.0
    pos = oracle.E4M3_TABLE[1:0x7F]
    assert np.all(np.diff(pos) > 0)               # codes 1..126 strictly increasing
    assert len(set(pos.tolist())) == 126
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0_value(255))


def test_mx_dequant_blocks():
    codes = np.array([[0x38] * 32 + [0x3C] * 32], dtype=np.uint8)
    scales = np.array([[127, 129]], dtype=np.uint8)
    v = oracle.mx_dequant(codes, scales)
    assert np.all(v[0, :32] == 1.0) and np.all(v[0, 32:] == 6.0)


# ---------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------
def _bwd_layer(seed, T=6, d=16, I=8, E=6, k=2, shared=True, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((d, E)) * 0.5
    b = rng.standard_normal(E) * 0.3 if bias else None
    experts = [(rng.standard_normal((I, d)) * 0.4, rng.standard_normal((I, d)) * 0.4,
                rng.standard_normal((d, I)) * 0.4) for _ in range(E)]
    sh = tuple(rng.standard_normal(s) * 0.4 for s in ((I, d), (I, d), (d, I))) if shared else None
    dy = rng.standard_normal((T, d))
    return x, wg, b, experts, sh, k, dy, rng


def _loss(x, wg, b, experts, sh, k, dy, **kw):
    f = oracle.layer(x, wg, b, experts, sh, k, **kw)
    return float((f["y"] * dy).sum()), f["ids"]


@pytest.mark.parametrize("mode", ["learned", "replay_gate_weights", "replay_caller_weights"])
def test_layer_backward_matches_central_differences(mode):
    """Every gradient against the derivative of the oracle's own forward along a random
    direction of each parameter group (central differences, eps = 1e-6; the expert
    choice is checked unchanged at both ends)."""
    x, wg, b, experts, sh, k, dy, rng = _bwd_layer(11)
    T, E = x.shape[0], wg.shape[1]
    kw = {}
    if mode != "learned":
        kw["ids_in"] = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    if mode == "replay_caller_weights":
        kw["weights_in"] = rng.dirichlet(np.ones(k), size=T)
    g = oracle.layer_backward(x, wg, b, experts, sh, k, dy, **kw)
    eps = 1e-6

    def check(name, grad, perturb):
        v = rng.standard_normal(grad.shape)
        lp, ip = _loss(*perturb(eps * v), k, dy, **kw)
        lm, im = _loss(*perturb(-eps * v), k, dy, **kw)
        assert np.array_equal(ip, im)
        fd = (lp - lm) / (2 * eps)
        an = float((grad * v).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)

    check("dx", g["dx"], lambda p: (x + p, wg, b, experts, sh))
    check("d_w_gate", g["d_w_gate"], lambda p: (x, wg + p, b, experts, sh))
    check("d_bias", g["d_bias"], lambda p: (x, wg, b + p, experts, sh))
    for e in range(E):
        for i, name in enumerate(("dw1", "dw3", "dw2")):
            def pert(p, e=e, i=i):
                ex = list(experts)
                m = list(ex[e])
                m[i] = m[i] + p
                ex[e] = tuple(m)
                return (x, wg, b, ex, sh)
            check(f"{name}[{e}]", g[name][e], pert)
    for i in range(3):
        def pert_s(p, i=i):
            m = list(sh)
            m[i] = m[i] + p
            return (x, wg, b, experts, tuple(m))
        check(f"shared[{i}]", g["d_shared"][i], pert_s)
    if mode == "replay_caller_weights":
        assert not g["d_w_gate"].any() and not g["d_bias"].any()


def test_backward_k1_has_no_gate_gradient_and_dense_form():
    """k = 1: the renormalised weight is 1 whatever the logits, so the gate gets no
    gradient; then dx is the dense sum of the chosen expert's and the shared expert's
    input gradients."""
    x, wg, b, experts, sh, _, dy, _ = _bwd_layer(12, k=1)
    g = oracle.layer_backward(x, wg, b, experts, sh, 1, dy)
    assert not g["d_w_gate"].any() and not g["d_bias"].any()
    ids = g["fwd"]["ids"][:, 0]
    for t in range(x.shape[0]):
        gx, *_ = oracle.expert_backward(x[t:t + 1], dy[t:t + 1], *experts[ids[t]])
        sx, *_ = oracle.expert_backward(x[t:t + 1], dy[t:t + 1], *sh)
        assert np.allclose(g["dx"][t], gx[0] + sx[0], rtol=1e-12, atol=1e-12)


def test_softmax_pick_grad_closed_form_k2():
    """k = 2: w0 = sigmoid(l0 - l1), so dl0 = w0 w1 (dw0 - dw1) = -dl1."""
    rng = np.random.default_rng(13)
    l = rng.standard_normal((20, 2))
    w = np.exp(l) / np.exp(l).sum(axis=1, keepdims=True)
    dw = rng.standard_normal((20, 2))
    dl = oracle.softmax_pick_grad(w, dw)
    ref = w[:, 0] * w[:, 1] * (dw[:, 0] - dw[:, 1])
    assert np.allclose(dl[:, 0], ref, rtol=0, atol=1e-15)
    assert np.allclose(dl[:, 1], -ref, rtol=0, atol=1e-15)


def test_silu_grad_values():
    assert oracle.silu_grad(0.0) == 0.5
    z = np.linspace(-8, 8, 33)
    h = 1e-6
    fd = (oracle.silu(z + h) - oracle.silu(z - h)) / (2 * h)
    assert np.allclose(oracle.silu_grad(z), fd, rtol=0, atol=1e-9)
    # large |z|: silu' -> 1 (z >> 0) and -> 0 (z << 0)
    assert abs(oracle.silu_grad(40.0) - 1.0) < 1e-15 and abs(oracle.silu_grad(-40.0)) < 1e-15


# ---------------------------------------------------------------------------
# NVFP4 quantization (E2M1 values, E4M3 scale per 16, fp32 scale per row)
# ---------------------------------------------------------------------------
def _brute_nearest(x, mags):
    """Index of the nearest magnitude, ties to the even index, by exhaustive search."""
    a = min(abs(x), mags[-1])
    best = None
    for i, m in enumerate(mags):
        dd = abs(a - m)
        if best is None or dd < best[0] or (dd == best[0] and i % 2 == 0):
            best = (dd, i)
    return best[1]


def test_e2m1_and_e4m3_rounding_brute_force():
    rng = np.random.default_rng(40)
    mags2 = list(oracle.E2M1_TABLE[:8])
    vals = list(rng.uniform(0, 7, 300)) + [0.5 * (a + b) for a, b in zip(mags2, mags2[1:])]
    vals += [v * (1 + s * 2.0 ** -20) for v in vals[-7:] for s in (-1, 1)]
    for v in vals:
        for sgn in (1.0, -1.0):
            c = int(oracle.e2m1_rne_codes([sgn * v])[0])
            assert c & 7 == _brute_nearest(v, mags2), v
            assert (c >> 3) == (1 if sgn < 0 else 0)
    mags3 = list(oracle.E4M3_TABLE[:127])
    vals = list(np.exp(rng.uniform(np.log(2.0 ** -11), np.log(500.0), 400)))
    vals += [0.5 * (a + b) for a, b in zip(mags3, mags3[1:])][::3]
    got = oracle.e4m3_rne_codes(vals)
    for v, c in zip(vals, got):
        assert int(c) == _brute_nearest(v, mags3), v


def test_e4m3_rounding_matches_an_independent_encoder():
    """The input generator's E4M3 encoder is separate code (integer bit manipulation)."""
    import torch
    import synth.inputs as si
    rng = np.random.default_rng(41)
    v = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 5000)).astype(np.float32)
    ref = si._e4m3_rne_codes(torch.from_numpy(v)).numpy().astype(np.uint8)
    assert np.array_equal(oracle.e4m3_rne_codes(v), ref)


def test_bf16_rne_matches_torch():
    import torch
    rng = np.random.default_rng(42)
    v = rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000))
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_rne(v.astype(np.float32).astype(np.float64)), ref)


def test_nvfp4_quantize_golden():
    g = json.load(open(os.path.join(GOLDEN, "nvfp4_hand.json")))
    v = np.asarray(g["rows"], dtype=np.float32)
    codes, sb, s = oracle.nvfp4_quantize(v)
    assert codes.tolist() == g["codes"]
    assert sb.tolist() == g["block_scales"]
    assert s.tolist() == g["row_scales"]
    assert np.array_equal(oracle.nvfp4_dequant(codes, sb, s), np.asarray(g["dequant"]))


def test_nvfp4_power_of_two_scaling_and_error_bound():
    rng = np.random.default_rng(43)
    v = _bf16_values(rng, (24, 64), scale=3.0)
    v[3] = 0.0                                  # a zero row
    v[5, :16] = 0.0                             # a zero block
    codes, sb, s = oracle.nvfp4_quantize(v)
    assert s[3] == 0 and not codes[3].any() and not sb[3].any()
    assert not codes[5, :16].any()
    # scaling a row by 2^j scales its row scale by 2^j and keeps every code
    for j in (-7, 5):
        c2, sb2, s2 = oracle.nvfp4_quantize(v * np.float32(2.0 ** j))
        assert np.array_equal(c2, codes) and np.array_equal(sb2, sb)
        assert np.array_equal(s2, s * np.float32(2.0 ** j))
    # each element is within half an E2M1 step (at its magnitude) of its block's grid
    deq = oracle.nvfp4_dequant(codes, sb, s)
    den = np.repeat(oracle.E4M3_TABLE[sb], 16, axis=1) * s[:, None]
    q = np.abs(v.astype(np.float64)) / np.where(den > 0, den, 1)
    gap = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
    err = np.abs(deq - v) / np.where(den > 0, den, 1)
    # (the quantizer divides in fp32: a relative 1e-6 covers values within an fp32 ulp of a tie)
    assert np.all((err <= gap / 2 * (1 + 1e-6)) | (q > 6))
    # a row's largest element lands on its block's top code (6) or one below
    assert np.all(np.abs(deq).max(axis=1)[s > 0] > 0)


def test_nvfp4_requantize_is_identity_and_layer_plumbing():
    rng = np.random.default_rng(44)
    v = _bf16_values(rng, (16, 48), scale=2.0)
    q = oracle.nvfp4_quantize(v)
    deq = oracle.nvfp4_dequant(*q).astype(np.float32)
    q2 = oracle.nvfp4_quantize(deq)          # the grid values quantize to themselves
    assert all(np.array_equal(a, b) for a, b in zip(q, q2))
    # identical experts: y_t = sum_r w_tr FFN(x_t) = FFN(x_t) (the weights sum to one)
    T, d, I, E, k = 6, 32, 32, 5, 2
    x = _bf16_values(rng, (T, d))
    wg = _f32(rng.standard_normal((d, E)))
    mats = [oracle.nvfp4_quantize(_bf16_values(rng, sh, 0.3)) for sh in ((I, d), (I, d), (d, I))]
    res = oracle.layer_nvfp4(x, wg, None, [tuple(mats)] * E, None, k)
    ref = oracle.expert_ffn_nvfp4(x, *mats)
    assert np.allclose(res["y"], ref, rtol=1e-12, atol=1e-12)


def test_nvfp4_expert_ffn_closed_form():
    """A case whose every step has a closed form.  Token t is c_t e_{j_t}; W1 holds one 2 per
    column (hidden unit pi(j) of input j), W3 is all ones, so a = 2 xq_t at unit pi(j_t) and
    0 elsewhere and g = xq_t at every unit: h has one nonzero per row, silu(2 xq) xq.  A row
    with a single nonzero v quantizes to code 6 under block scale 448, i.e. to
    sign(v) 2688 fl32(|v| / 2688).  So y[t, o] = Q(bf16(silu(2 xq) xq)) W2[o, pi(j_t)] with
    xq = Q(c_t).  (d = I, so a transposed W2 would go unnoticed by shapes alone.)"""
    import torch
    d = I = 32
    rng = np.random.default_rng(45)
    pi = rng.permutation(I)
    one = 0x38                                        # E4M3 code of 1.0
    code_of = {0.0: 0, 1.0: 2, 2.0: 4, 6.0: 7}        # E2M1 magnitudes -> codes
    w1c = np.zeros((I, d), np.uint8)
    w1c[pi, np.arange(d)] = code_of[2.0]              # W1[pi(j), j] = 2
    w1 = (w1c, np.full((I, d // 16), one, np.uint8), np.ones(I, np.float32))
    w3 = (np.full((I, d), code_of[1.0], np.uint8), np.full((I, d // 16), one, np.uint8), np.ones(I, np.float32))
    w2 = (rng.integers(0, 16, (d, I)).astype(np.uint8), rng.integers(0x20, 0x48, (d, I // 16)).astype(np.uint8),
          rng.uniform(0.5, 2.0, d).astype(np.float32))
    W2 = oracle.nvfp4_dequant(*w2)

    def q1(v):                                        # NVFP4 value of a row's only nonzero
        return np.sign(v) * 2688.0 * float(np.float32(abs(v)) / np.float32(2688.0))

    cs = [1.0, -0.75, 2.5, 0.3125, -3.0, 0.0390625]
    js = rng.integers(0, d, len(cs))
    x = np.zeros((len(cs), d), np.float32)
    x[np.arange(len(cs)), js] = cs
    y = oracle.expert_ffn_nvfp4(x, w1, w3, w2)
    for t, (c, j) in enumerate(zip(cs, js)):
        xq = q1(c)
        h = (2 * xq) / (1 + np.exp(-2 * xq)) * xq
        hb = float(torch.tensor(h, dtype=torch.float64).float().bfloat16().double())
        ref = q1(hb) * W2[:, pi[j]]
        assert np.allclose(y[t], ref, rtol=1e-13, atol=0), t


# ---------------------------------------------------------------------------
# MXFP8 quantiser and the MXFP8 backward
# ---------------------------------------------------------------------------
FINITE_E4M3 = sorted(set(abs(v) for v in oracle.E4M3_TABLE.tolist() if not math.isnan(v)))


def _mx_brute(block):
    """Smallest power of two X with amax / X <= 448 by search, then every element the
    nearest grid value (ties: the even code, i.e. the grid index that is even)."""
    amax = max(abs(v) for v in block)
    if amax == 0:
        return [0.0] * len(block)
    e = -200
    while amax / 2.0 ** e > 448.0:
        e += 1
    X = 2.0 ** e
    out = []
    for v in block:
        q = abs(v) / X
        best = min(range(len(FINITE_E4M3)), key=lambda i: (abs(FINITE_E4M3[i] - q), i % 2))
        out.append(math.copysign(FINITE_E4M3[best] * X, v) if FINITE_E4M3[best] else 0.0)
    return out


def test_mx_quantize_brute_force_and_scale_rule():
    rng = np.random.default_rng(60)
    rows = [rng.standard_normal(32) * s for s in (1e-3, 0.3, 1.0, 7.0, 900.0, 2.0 ** -60)]
    mids = [(a + b) / 2 for a, b in zip(FINITE_E4M3[1:-1], FINITE_E4M3[2:])]
    tie = np.array(mids[:31] + [448.0])             # exact midpoints: ties to even
    rows += [tie, -tie, tie * 2.0 ** -5]
    sat = np.full(32, 0.5)
    sat[0] = 449.0 / 448.0 * 2.0 ** 8               # amax / 2^(floor log2 - 8) > 448: next power
    rows += [sat, np.zeros(32)]
    v = np.stack(rows)
    q = oracle.mx_quantize(v)
    for r in range(len(rows)):
        want = _mx_brute(list(v[r]))
        assert np.array_equal(q[r], np.array(want)), r
    # the block maximum keeps its magnitude up to half a step: no element saturates
    # (449/448 * 2^8 takes X = 2: 128.3 -> 128, not X = 1, which would clamp to 448)
    assert q[len(rows) - 2][0] == 256.0
    assert oracle.mx_quantize(np.zeros((2, 64))).tolist() == np.zeros((2, 64)).tolist()


def test_mx_quantize_round_trip_scaling_and_axis():
    rng = np.random.default_rng(61)
    v = rng.standard_normal((8, 96)) * 3
    q = oracle.mx_quantize(v)
    assert np.array_equal(oracle.mx_quantize(q), q)                    # representable: unchanged
    for s in (-7, 3, 20):
        assert np.array_equal(oracle.mx_quantize(v * 2.0 ** s), q * 2.0 ** s)
    assert np.array_equal(oracle.mx_quantize(v.T, axis=0), q.T)
    err = np.abs(q - v)
    X = np.repeat(2.0 ** np.ceil(np.log2(np.abs(v).reshape(8, 3, 32).max(-1) / 448)), 32, axis=1)
    assert np.all(err <= X * 2.0 ** -4 * np.maximum(np.abs(q) / X, 2.0 ** -6) * 2)   # half an E4M3 step


def _mx_layer(seed, T=40, d=64, I=32, E=6, k=2, shared=True, bias=True):
    rng = np.random.default_rng(seed)
    x = oracle.mx_quantize(rng.standard_normal((T, d)))
    wg = rng.standard_normal((d, E)) / 8
    b = rng.standard_normal(E) * 0.3 if bias else None
    mk = lambda *s: oracle.mx_quantize(rng.standard_normal(s) / np.sqrt(s[-1]))  # noqa: E731
    experts = [(mk(I, d), mk(I, d), mk(d, I)) for _ in range(E)]
    sh = (mk(I, d), mk(I, d), mk(d, I)) if shared else None
    dy = rng.standard_normal((T, d))
    return x, wg, b, experts, sh, k, dy, rng


def test_layer_mxfp8_identity_projections_give_the_quantised_h():
    """With W1 = W3 = W2 = the identity (d = I = 32), k = 1 (weight exactly 1) and both
    experts equal, y = MX(silu(x) x) row by row: the forward multiplies the per-row MXFP8
    requantisation of h.  It differs from the exact h, and one token alone gives its row
    of the batch (the quantisation never mixes tokens)."""
    rng = np.random.default_rng(71)
    T, d, E = 9, 32, 2
    x = oracle.mx_quantize(rng.standard_normal((T, d)) * 2.0)
    wg = rng.standard_normal((d, E))
    eye = np.eye(d)
    experts = [(eye, eye, eye)] * E
    y = oracle.layer_mxfp8(x, wg, None, experts, None, 1)["y"]
    h = x * x / (1.0 + np.exp(-x))
    assert np.array_equal(y, oracle.mx_quantize(h, axis=1))
    assert not np.array_equal(y, h)
    for t in (0, 4, 8):
        one = oracle.layer_mxfp8(x[t:t + 1], wg, None, experts, None, 1)["y"]
        assert np.array_equal(one[0], y[t])


@pytest.mark.parametrize("mode", ["learned", "replay"])
def test_layer_mxfp8_is_the_mxfp8_backward_forward_and_layer_without_quantisation(mode):
    """The forward of ``layer_backward_mxfp8`` (an independent loop over the same
    readings) gives the same y bit for bit; with an identity quantiser the layer is the
    unquantised ``layer``, bit for bit, with the same routing and dispatch."""
    x, wg, b, experts, sh, k, dy, rng = _mx_layer(64)
    T, E = x.shape[0], wg.shape[1]
    kw = {} if mode == "learned" else {"ids_in": np.stack([rng.permutation(E)[:k] for _ in range(T)])}
    f = oracle.layer_mxfp8(x, wg, b, experts, sh, k, **kw)
    g = oracle.layer_backward_mxfp8(x, wg, b, experts, sh, k, dy, **kw)
    assert np.array_equal(f["y"], g["y"])
    ident = lambda v, axis=-1: np.asarray(v, float)  # noqa: E731
    u = oracle.layer_mxfp8(x, wg, b, experts, sh, k, quant=ident, **kw)
    ref = oracle.layer(x, wg, b, experts, sh, k, **kw)
    assert np.array_equal(u["y"], ref["y"])
    for n in ("ids", "weights", "offsets", "perm", "row_of"):
        assert np.array_equal(u[n], ref[n]) and np.array_equal(f[n], ref[n]), n
    # the quantised h moves y by a few percent of its size, not more
    rel = float(np.linalg.norm(f["y"] - ref["y"]) / np.linalg.norm(ref["y"]))
    assert 1e-3 < rel < 0.1, rel


@pytest.mark.parametrize("mode", ["learned", "replay_gate_weights", "replay_caller_weights"])
def test_mxfp8_backward_without_quantisation_is_the_exact_chain_rule(mode):
    x, wg, b, experts, sh, k, dy, rng = _mx_layer(62)
    T, E = x.shape[0], wg.shape[1]
    kw = {}
    if mode != "learned":
        kw["ids_in"] = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    if mode == "replay_caller_weights":
        kw["weights_in"] = rng.dirichlet(np.ones(k), size=T)
    ident = lambda v, axis=-1: np.asarray(v, float)  # noqa: E731
    g = oracle.layer_backward_mxfp8(x, wg, b, experts, sh, k, dy, quant=ident, grad_round=ident, **kw)
    ref = oracle.layer_backward(x, wg, b, experts, sh, k, dy, dense=False, **kw)
    rel = lambda a, r: float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-300))  # noqa: E731
    assert rel(g["y"], ref["fwd"]["y"]) < 1e-12
    for n in ("dx", "d_weights", "d_w_gate"):
        assert rel(g[n], ref[n]) < 1e-12, n
    for n in ("dw1", "dw3", "dw2"):
        assert set(g[n]) == set(ref[n])
        for e in g[n]:
            assert rel(g[n][e], ref[n][e]) < 1e-12, (n, e)
    for i in range(3):
        assert rel(g["d_shared"][i], ref["d_shared"][i]) < 1e-12


def test_mxfp8_backward_quantisation_axes():
    """A power-of-two scaling S commutes with MX quantisation of the scaled values, and
    S = 2^16 pushes the other elements of a block it shares with them below the E4M3
    range, so each check holds only with the right axis: (1) one token's dy times S scales
    that token's dx by S and leaves every other token's dx as it was (data gradients
    quantised per row); (2) one column of every W2 times S scales that column of dL/dh by
    S and no other (W2 requantised along d); (3) one column of dy times S scales that row
    of every dW2 by S and no other (weight-gradient operands quantised along the rows);
    (4) with that input feature zero in x and caller weights, one column of W1 and W3
    times S scales that column of dx by S and no other (W1, W3 requantised along I)."""
    x, wg, b, experts, sh, k, dy, rng = _mx_layer(63)
    T, E = x.shape[0], wg.shape[1]
    S = 2.0 ** 16
    g0 = oracle.layer_backward_mxfp8(x, wg, b, experts, sh, k, dy)
    # the forward's h is quantised per row along I: its rows are MX values already
    assert np.array_equal(oracle.mx_quantize(g0["hq_rows"]), g0["hq_rows"])
    # (1)
    dy1 = dy.copy()
    dy1[7] *= S
    g1 = oracle.layer_backward_mxfp8(x, wg, b, experts, sh, k, dy1)
    others = np.arange(T) != 7
    assert np.array_equal(g1["dx"][others], g0["dx"][others])
    assert np.array_equal(g1["dx"][7], S * g0["dx"][7])
    # (2)
    n0 = 5
    ex2 = [(a, c, w2.copy()) for a, c, w2 in experts]
    for _, _, w2 in ex2:
        w2[:, n0] *= S
    sh2 = (sh[0], sh[1], sh[2].copy())
    sh2[2][:, n0] *= S
    g2 = oracle.layer_backward_mxfp8(x, wg, b, ex2, sh2, k, dy)
    keep = np.arange(g0["dh_rows"].shape[1]) != n0
    assert np.array_equal(g2["dh_rows"][:, keep], g0["dh_rows"][:, keep])
    assert np.array_equal(g2["dh_rows"][:, n0], S * g0["dh_rows"][:, n0])
    # (3)
    c0 = 11
    dy3 = dy.copy()
    dy3[:, c0] *= S
    g3 = oracle.layer_backward_mxfp8(x, wg, b, experts, sh, k, dy3)
    rows = np.arange(dy.shape[1]) != c0
    for e in g0["dw2"]:
        assert np.array_equal(g3["dw2"][e][rows], g0["dw2"][e][rows])
        assert np.array_equal(g3["dw2"][e][c0], S * g0["dw2"][e][c0])
    # (4)
    i0 = 9
    x4 = x.copy()
    x4[:, i0] = 0.0
    kw = {"ids_in": g0["ids"], "weights_in": g0["weights"]}
    g4a = oracle.layer_backward_mxfp8(x4, wg, b, experts, sh, k, dy, **kw)
    ex4 = [(w1.copy(), w3.copy(), w2) for w1, w3, w2 in experts]
    for w1, w3, _ in ex4:
        w1[:, i0] *= S
        w3[:, i0] *= S
    sh4 = (sh[0].copy(), sh[1].copy(), sh[2])
    sh4[0][:, i0] *= S
    sh4[1][:, i0] *= S
    g4b = oracle.layer_backward_mxfp8(x4, wg, b, ex4, sh4, k, dy, **kw)
    cols = np.arange(x.shape[1]) != i0
    assert np.array_equal(g4b["dx"][:, cols], g4a["dx"][:, cols])
    assert np.array_equal(g4b["dx"][:, i0], S * g4a["dx"][:, i0])


def test_mxfp8_backward_rounds_the_expert_output_gradient_to_bf16():
    """With W2 = the identity (d = I) and no MX quantisation, dL/dh of a dispatched row is
    its expert-output gradient itself: it must be w_tr dy_t rounded to bf16 (and differ
    from the unrounded product somewhere), the shared rows dy exactly."""
    rng = np.random.default_rng(64)
    T, d, E, k = 12, 32, 4, 2
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((d, E)) / 4
    eye = np.eye(d)
    experts = [(rng.standard_normal((d, d)) / 6, rng.standard_normal((d, d)) / 6, eye) for _ in range(E)]
    sh = (rng.standard_normal((d, d)) / 6, rng.standard_normal((d, d)) / 6, eye)
    dy = oracle.bf16_rne(rng.standard_normal((T, d)))
    ident = lambda v, axis=-1: np.asarray(v, float)  # noqa: E731
    g = oracle.layer_backward_mxfp8(x, wg, None, experts, sh, k, dy, quant=ident)
    dh = g["dh_rows"]
    assert np.array_equal(oracle.bf16_rne(dh), dh)
    raw = np.stack([g["weights"][t, r] * dy[t] for t in range(T) for r in range(k)])
    rows = np.array([g["row_of"][t * k + r] for t in range(T) for r in range(k)])
    assert np.array_equal(dh[rows], oracle.bf16_rne(raw))
    assert np.any(dh[rows] != raw)
    assert np.array_equal(dh[T * k:], dy)


def test_mxfp8_backward_of_the_nvfp4_forward():
    """With forward="nvfp4" the backward's forward is the pinned NVFP4 layer (same ids and
    y, the same expert outputs), and the expert forward hands the MXFP8 backward (pinned
    above) the x the NVFP4 forward multiplied: its per-row NVFP4 values."""
    rng = np.random.default_rng(65)
    T, d, I, E, k = 24, 64, 32, 4, 2
    x = _bf16_values(rng, (T, d))
    wg = rng.standard_normal((d, E)) / 6
    b = rng.standard_normal(E) * 0.2
    mk = lambda *sh: oracle.nvfp4_quantize(_bf16_values(rng, sh, 1 / np.sqrt(sh[-1])))  # noqa: E731
    experts = [(mk(I, d), mk(I, d), mk(d, I)) for _ in range(E)]
    sh = (mk(I, d), mk(I, d), mk(d, I))
    dy = oracle.bf16_rne(rng.standard_normal((T, d)))
    g = oracle.layer_backward_mxfp8(x, wg, b, experts, sh, k, dy, forward="nvfp4")
    ref = oracle.layer_nvfp4(x, wg, b, experts, sh, k)
    assert np.array_equal(g["ids"], ref["ids"])
    assert np.max(np.abs(g["y"] - ref["y"])) <= 1e-12 * np.max(np.abs(ref["y"]))
    xq, _, _, _, out, _ = oracle.expert_forward_nvfp4(x[:5], *experts[1])
    assert np.array_equal(out, oracle.expert_ffn_nvfp4(x[:5], *experts[1]))
    assert np.array_equal(xq, oracle.nvfp4_dequant(*oracle.nvfp4_quantize(np.asarray(x[:5], np.float32))))
    for e in g["dw1"]:
        assert g["dw1"][e].shape == (I, d) and g["dw2"][e].shape == (d, I)
