"""CPU oracle of one Mixture-of-Experts layer's forward and backward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the library never does, and
it shares no code with the HIP path (the seeded input generator aside, which
holds none of this arithmetic).

What it computes, and where that is defined:
  * A gating layer picks, for each token, 8 of 384 experts from the token's hidden
    state (Training Data podcast page "How Cursor Trained Composer on Fireworks",
    section on floating point and MoE; same fact on the page "Cursor 訓練 Composer 2
    的五大工程挑戰", section "浮點數的陷阱").  The pages do not state the gating
    function; the reading used here is softmax over all experts, keep the top k,
    renormalise the kept probabilities to sum to one, ties to the lower index.
  * Router replay: the inference engine returns the chosen expert IDs per token per
    MoE layer and the training forward overrides the router's assignment with them,
    while the router still computes gate scores (Composer 2 Technical Report, §6.2,
    paragraph on inference and weight sync).
  * The experts run as one grouped GEMM per expert group (Composer 2 Technical
    Report, §6.1 "Kernels", Figure 10); each expert is a SwiGLU FFN
    (silu(x W1) * (x W3)) W2; the tokens' expert outputs are combined as the
    routing-weighted sum (§6.1 "Parallelism": dispatch and combine), plus the
    always-on shared expert when present.
  * The backward pass (the MoE layer is trained with grouped GEMMs forward and
    backward: Composer 2 Technical Report, §6.1 "Kernels", Figure 10; under replay
    the router still computes gate scores so that gradients flow through them:
    §6.2, paragraph on inference and weight sync): the chain rule of the forward
    above, in float64, for a scalar loss with dL/dy given.

Precision: every input value is converted to float64 exactly.  Gate logits are the
correctly rounded value of the exact sum (each product of two stored values is
exact in float64: at most 24 + 24 significant bits and no underflow for fp32, bf16
or MXFP8 inputs; ``math.fsum`` then rounds the exact sum once).  Selection uses
those exact logits.  Everything after selection is ordinary float64 (numpy).

Every function here is pinned by a CPU test against something other than itself
(closed forms, brute force, exact rational arithmetic, an independent
formulation); none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np


def f64(a) -> np.ndarray:
    """Exact conversion of stored values (fp32, bf16-as-fp32, ints) to float64."""
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# MXFP8 decoding (OCP Microscaling Formats v1.0: E4M3 elements, E8M0 scales)
# ---------------------------------------------------------------------------
def e4m3_value(code: int) -> float:
    """Value of one FP8 E4M3 code: sign, 4-bit exponent (bias 7), 3-bit mantissa.

    Exponent field 0 holds subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no
    infinities, so S.1111.110 = 448 is the largest magnitude.
    """
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        v = (m / 8.0) * 2.0 ** -6
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def e8m0_value(code: int) -> float:
    """Value of one E8M0 scale code: 2^(code - 127); code 255 is NaN."""
    if code == 255:
        return math.nan
    return 2.0 ** (int(code) - 127)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def mx_dequant(codes, scales, block: int = 32) -> np.ndarray:
    """Exact float64 values of an MXFP8 tensor stored along its last dimension."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    K = codes.shape[-1]
    assert scales.shape[-1] * block == K
    vals = E4M3_TABLE[codes]
    sc = E8M0_TABLE[scales]
    return vals * np.repeat(sc, block, axis=-1)


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------
def exact_logits(x, w_gate, bias=None) -> np.ndarray:
    """logit[t, e] = sum_i x[t, i] * w_gate[i, e] (+ bias[e]), correctly rounded.

    x [T, d], w_gate [d, E], bias [E] or None.  Each product is exact in float64
    (see the module docstring), and ``math.fsum`` returns the exact sum rounded
    once, so the result does not depend on any summation order.
    """
    x = f64(x)
    w = f64(w_gate)
    T, d = x.shape
    d2, E = w.shape
    assert d == d2
    assert np.all(np.isfinite(x)) and np.all(np.isfinite(w))
    b = None if bias is None else f64(bias)
    out = np.empty((T, E), dtype=np.float64)
    for t in range(T):
        prods = x[t][:, None] * w          # [d, E], every entry exact
        for e in range(E):
            terms = prods[:, e].tolist()
            if b is not None:
                terms.append(float(b[e]))
            out[t, e] = math.fsum(terms)
    return out


def topk_ids(logits, k: int) -> np.ndarray:
    """The k largest logits of each row, ordered by (logit descending, index ascending)."""
    logits = f64(logits)
    T, E = logits.shape
    assert 1 <= k <= E
    ids = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        row = logits[t]
        order = sorted(range(E), key=lambda e: (-row[e], e))
        ids[t] = order[:k]
    return ids


def softmax_pick_renormalise(logits, ids) -> np.ndarray:
    """Softmax over all experts, keep the probabilities at ``ids``, renormalise them.

    Rows of the result sum to one; column r is the weight of expert ids[t, r].
    """
    logits = f64(logits)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p = p / p.sum(axis=1, keepdims=True)
    picked = np.take_along_axis(p, np.asarray(ids, dtype=np.int64), axis=1)
    return picked / picked.sum(axis=1, keepdims=True)


def route(x, w_gate, bias, k: int):
    """Learned routing: returns (ids [T,k], weights [T,k] float64, logits [T,E])."""
    logits = exact_logits(x, w_gate, bias)
    ids = topk_ids(logits, k)
    return ids, softmax_pick_renormalise(logits, ids), logits


def route_certified(x, w_gate, bias, k: int):
    """Learned routing for large batches: the ids of ``route`` without an exact sum
    for every logit.

    1. L = x @ w_gate (+ bias) by an fp64 matrix product, summed in whatever order
       the BLAS library uses.  Each product of two stored values is exact (module
       docstring), so only the d additions (the bias included) round, and
       |L - l| <= gamma_{d+1} S with S = sum_i |x_i w_ie| + |b_e|,
       gamma_n = n u / (1 - n u), u = 2^-53 (the inner-product error bound of
       Higham, Accuracy and Stability of Numerical Algorithms, section 3.1, which
       holds for any summation order; d + 1 terms need only d additions).  The correctly rounded
       logit is within u |l| <= u S of the exact sum l.  B = 2 (gamma_{d+1} + u) S
       therefore bounds |L - fl(l)| twice over; the factor 2 also absorbs the
       rounding of S itself and of the comparisons below.
    2. A token is certified when the bounds separate its top-k order: every pair of
       adjacent ranks a, b among the first k has L_a - B_a > L_b + B_b, and rank k-1
       has L - B above L + B of every expert outside the first k.  Then the correctly
       rounded logits are strictly ordered the same way, so the ids (order included)
       are those of ``route``.
    3. Every other token gets ``exact_logits`` and ``topk_ids``, as in ``route``.
    Returns (ids [T, k], weights [T, k], n_exact): weights by
    ``softmax_pick_renormalise`` on L for certified tokens (they differ from
    ``route``'s by at most a few times max B, about 1e-10 at d = 7168) and on the exact
    logits for the others; n_exact = the number of tokens recomputed exactly.
    """
    x = f64(x)
    w = f64(w_gate)
    T, d = x.shape
    d2, E = w.shape
    assert d == d2 and 1 <= k <= E
    assert np.all(np.isfinite(x)) and np.all(np.isfinite(w))
    b = np.zeros(E) if bias is None else f64(bias)
    L = x @ w + b
    S = np.abs(x) @ np.abs(w) + np.abs(b)
    u = 2.0 ** -53
    gam = (d + 1) * u / (1 - (d + 1) * u)
    B = 2.0 * (gam + u) * S
    order = np.argsort(-L, axis=1, kind="stable")          # (L desc, index asc)
    top = order[:, :k]
    Lt = np.take_along_axis(L, top, axis=1)
    Bt = np.take_along_axis(B, top, axis=1)
    lo, hi = Lt - Bt, Lt + Bt
    ok = np.all(lo[:, :-1] > hi[:, 1:], axis=1)
    if k < E:
        rest = order[:, k:]
        rest_hi = np.max(np.take_along_axis(L, rest, axis=1) + np.take_along_axis(B, rest, axis=1), axis=1)
        ok &= lo[:, -1] > rest_hi
    ids = top.astype(np.int64)
    weights = softmax_pick_renormalise(L, ids)
    bad = np.nonzero(~ok)[0]
    for t in bad:
        lt = exact_logits(x[t:t + 1], w, bias)
        ids[t] = topk_ids(lt, k)[0]
        weights[t] = softmax_pick_renormalise(lt, ids[t:t + 1])[0]
    return ids, weights, len(bad)


def validate_replay_ids(ids_in, E: int) -> None:
    """Replayed IDs must lie in [0, E) and be distinct within each row."""
    ids = np.asarray(ids_in)
    if ids.ndim != 2:
        raise ValueError("replayed ids must be [T, k]")
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("replayed expert id out of range")
    for t in range(ids.shape[0]):
        if len(set(ids[t].tolist())) != ids.shape[1]:
            raise ValueError(f"replayed ids of token {t} are not distinct")


def route_replay(x, w_gate, bias, ids_in, weights_in=None):
    """Replayed routing: the caller's IDs override the router's choice.

    The gate logits are still computed.  Weights are the caller's (used verbatim)
    when given, else the router's softmax probabilities at the replayed IDs,
    renormalised, in the caller's column order.  Returns (ids, weights, logits).
    """
    logits = exact_logits(x, w_gate, bias)
    E = logits.shape[1]
    validate_replay_ids(ids_in, E)
    ids = np.asarray(ids_in, dtype=np.int64)
    if weights_in is not None:
        w = f64(weights_in).copy()
    else:
        w = softmax_pick_renormalise(logits, ids)
    return ids, w, logits


def route_replay_filtered(x, w_gate, bias, ids_in, log_tau: float):
    """Router replay with the plausibility filter.

    Composer 2 Technical Report, §6.2, paragraph on inference and weight sync: a
    replayed expert whose gate score falls below a plausibility threshold derived from
    the router's own top-k choice is dropped and replaced with the router's
    candidates.  The page fixes neither the score nor the threshold; the reading here:
      * score = the router's softmax probability p_e; threshold = tau * p_(k), where
        p_(k) is the probability of the router's own k-th choice (k = row width of
        ids_in) and tau >= 0 is the caller's parameter;
      * p_e >= tau p_(k) is tested in logit form, l_e - l_(k) >= ln tau, on the
        correctly rounded logits, the difference rounded once in float64; the caller
        passes ln tau (-inf keeps every replayed id: plain replay; +inf drops all:
        learned routing);
      * dropped columns are refilled, in column order, by the router's top-k ids in
        rank order that are not among the kept replayed ids;
      * weights: the router's softmax probabilities at the final ids, renormalised,
        in column order (as for replay without caller weights).
    Returns (ids, weights, keep [T, k] bool, logits).
    """
    logits = exact_logits(x, w_gate, bias)
    T, E = logits.shape
    validate_replay_ids(ids_in, E)
    q = np.asarray(ids_in, dtype=np.int64)
    k = q.shape[1]
    lt = float(log_tau)
    if math.isnan(lt):
        raise ValueError("log_tau is NaN")
    router = topk_ids(logits, k)
    ids = np.empty((T, k), dtype=np.int64)
    keep = np.zeros((T, k), dtype=bool)
    for t in range(T):
        lk = float(logits[t, router[t, k - 1]])
        for j in range(k):
            keep[t, j] = (float(logits[t, q[t, j]]) - lk) >= lt
        kept = {int(e) for e, kp in zip(q[t], keep[t]) if kp}
        fill = [int(e) for e in router[t] if int(e) not in kept]
        for j in range(k):
            ids[t, j] = q[t, j] if keep[t, j] else fill.pop(0)
    return ids, softmax_pick_renormalise(logits, ids), keep, logits


# ---------------------------------------------------------------------------
# Dispatch (token permutation into contiguous per-expert segments)
# ---------------------------------------------------------------------------
def dispatch(ids, E: int):
    """Sort the T*k (token, slot) pairs by (expert ascending, token ascending).

    Returns offsets [E+1] (segment e is rows offsets[e]..offsets[e+1]-1),
    perm [T*k] with perm[j] = t*k + r for sorted row j, and row_of [T*k] with
    row_of[t*k + r] = j (the inverse of perm).
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    pairs = sorted((int(ids[t, r]), t, r) for t in range(T) for r in range(k))
    counts = [0] * E
    for e, _, _ in pairs:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.array([t * k + r for (_, t, r) in pairs], dtype=np.int64)
    row_of = np.empty(T * k, dtype=np.int64)
    row_of[perm] = np.arange(T * k)
    return offsets, perm, row_of


# ---------------------------------------------------------------------------
# Expert FFN and combine
# ---------------------------------------------------------------------------
def silu(z):
    """silu(z) = z / (1 + exp(-z)) = z * sigmoid(z)."""
    z = f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(x_rows, w1, w3, w2) -> np.ndarray:
    """SwiGLU expert: (silu(x W1) * (x W3)) W2 in float64.

    Weights are stored output-major: w1, w3 [I, d] and w2 [d, I], so the
    mathematical W1 is ``w1.T``.
    """
    xr = f64(x_rows)
    a = xr @ f64(w1).T
    g = xr @ f64(w3).T
    return (silu(a) * g) @ f64(w2).T


def layer(x, w_gate, bias, experts, shared, k: int, ids_in=None, weights_in=None):
    """One MoE layer forward through dispatch, per-expert FFN and combine.

    ``experts[e]`` -> (w1, w3, w2) for routed expert e (any indexable; it may fetch
    lazily); ``shared`` is (w1, w3, w2) or None.  With ``ids_in`` the routing is
    replayed.  Returns a dict with y [T, d] and the routing/dispatch intermediates.
    """
    xf = f64(x)
    T, d = xf.shape
    if ids_in is None:
        ids, w, logits = route(xf, w_gate, bias, k)
    else:
        ids, w, logits = route_replay(xf, w_gate, bias, ids_in, weights_in)
    E = logits.shape[1]
    offsets, perm, row_of = dispatch(ids, E)
    rows = np.zeros((T * k, d), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = perm[lo:hi] // k
        w1, w3, w2 = experts[e]
        rows[lo:hi] = expert_ffn(xf[toks], w1, w3, w2)
    y = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        for r in range(k):
            y[t] += w[t, r] * rows[row_of[t * k + r]]
    if shared is not None:
        y += expert_ffn(xf, *shared)
    return {"y": y, "ids": ids, "weights": w, "logits": logits,
            "offsets": offsets, "perm": perm, "row_of": row_of, "rows": rows}


def layer_dense(x, w_gate, bias, experts, shared, k: int):
    """The same layer without dispatch: y = sum_e g_e(x) FFN_e(x) + shared(x).

    g_e is the routing weight if e was selected for the token, else 0.  Every
    expert runs on every token, so this form never permutes anything.
    """
    xf = f64(x)
    T, d = xf.shape
    ids, w, logits = route(xf, w_gate, bias, k)
    E = logits.shape[1]
    G = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for r in range(k):
            G[t, ids[t, r]] = w[t, r]
    y = np.zeros((T, d), dtype=np.float64)
    for e in range(E):
        if not np.any(G[:, e]):
            continue
        y += G[:, e:e + 1] * expert_ffn(xf, *experts[e])
    if shared is not None:
        y += expert_ffn(xf, *shared)
    return y


def normwise_rel_err(y, y_ref) -> float:
    """max |y - y_ref| / max |y_ref| over all elements compared."""
    y = f64(y)
    y_ref = f64(y_ref)
    den = np.max(np.abs(y_ref))
    if den == 0:
        return float(np.max(np.abs(y)))
    return float(np.max(np.abs(y - y_ref)) / den)


# ---------------------------------------------------------------------------
# Backward pass of the layer (gradients of a scalar loss L with dL/dy = dy)
# ---------------------------------------------------------------------------
def silu_grad(z):
    """d silu / dz = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    z = f64(z)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def expert_backward(x_rows, d_out_rows, w1, w3, w2):
    """Chain rule through one SwiGLU expert o = (silu(a) * g) W2, a = x W1, g = x W3.

    x_rows [n, d], d_out_rows = dL/do [n, d]; weights stored output-major (w1, w3
    [I, d], w2 [d, I]).  Returns (dx [n, d], dw1 [I, d], dw3 [I, d], dw2 [d, I]).
    """
    xr = f64(x_rows)
    do = f64(d_out_rows)
    w1, w3, w2 = f64(w1), f64(w3), f64(w2)
    a = xr @ w1.T
    g = xr @ w3.T
    h = silu(a) * g
    dh = do @ w2                      # dL/dh [n, I]
    dg = dh * silu(a)
    da = dh * g * silu_grad(a)
    dx = da @ w1 + dg @ w3
    return dx, da.T @ xr, dg.T @ xr, do.T @ h


def softmax_pick_grad(weights, d_weights):
    """dL/dl at the chosen experts for w = exp(l_S) / sum exp(l_S) (the softmax over
    all experts, picked at S and renormalised, depends only on the logits in S):
    dl_r = w_r (dw_r - sum_s w_s dw_s)."""
    w = f64(weights)
    dw = f64(d_weights)
    return w * (dw - (w * dw).sum(axis=1, keepdims=True))


def layer_backward(x, w_gate, bias, experts, shared, k: int, dy, ids_in=None, weights_in=None,
                   dense: bool = True):
    """Gradients of L = <dy, y> through one MoE layer forward (``layer``).

    The expert choice is piecewise constant in x, so no gradient flows through the
    selection; the gate's logits get one through the routing weights whenever those
    come from the gate (learned routing, or replay without caller weights; the
    router still computes gate scores so that gradients can flow through it:
    Composer 2 Technical Report, §6.2, paragraph on inference and weight sync).
    Returns a dict: dx [T, d], d_weights [T, k], d_w_gate [d, E], d_bias [E] (or
    None), dw1 / dw3 [E, I, d], dw2 [E, d, I], d_shared (dw1, dw3, dw2) or None, and
    the forward dict under "fwd".  With dense=False the expert gradients are dicts
    holding only the experts that got rows (the others are zero).
    """
    xf = f64(x)
    dyf = f64(dy)
    fwd = layer(xf, w_gate, bias, experts, shared, k, ids_in=ids_in, weights_in=weights_in)
    T, d = xf.shape
    E = fwd["logits"].shape[1]
    ids, w, rows = fwd["ids"], fwd["weights"], fwd["rows"]
    offsets, perm, row_of = fwd["offsets"], fwd["perm"], fwd["row_of"]
    # combine: y_t = sum_r w_tr o_tr (+ shared_t)
    d_weights = np.empty((T, k))
    d_rows = np.empty_like(rows)
    for t in range(T):
        for r in range(k):
            j = row_of[t * k + r]
            d_weights[t, r] = float(dyf[t] @ rows[j])
            d_rows[j] = w[t, r] * dyf[t]
    dx = np.zeros((T, d))
    if dense:
        I = f64(experts[0][0]).shape[0]
        dw1 = np.zeros((E, I, d))
        dw3 = np.zeros((E, I, d))
        dw2 = np.zeros((E, d, I))
    else:
        dw1, dw3, dw2 = {}, {}, {}
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = perm[lo:hi] // k
        gx, dw1[e], dw3[e], dw2[e] = expert_backward(xf[toks], d_rows[lo:hi], *experts[e])
        np.add.at(dx, toks, gx)
    d_shared = None
    if shared is not None:
        gx, s1, s3, s2 = expert_backward(xf, dyf, *shared)
        dx += gx
        d_shared = (s1, s3, s2)
    d_w_gate = np.zeros((d, E))
    d_bias = None if bias is None else np.zeros(E)
    if weights_in is None:   # weights are the gate's softmax at the chosen ids
        dl = softmax_pick_grad(w, d_weights)
        wg = f64(w_gate)
        for t in range(T):
            for r in range(k):
                e = int(ids[t, r])
                dx[t] += dl[t, r] * wg[:, e]
                d_w_gate[:, e] += dl[t, r] * xf[t]
                if d_bias is not None:
                    d_bias[e] += dl[t, r]
    return {"dx": dx, "d_weights": d_weights, "d_w_gate": d_w_gate, "d_bias": d_bias,
            "dw1": dw1, "dw3": dw3, "dw2": dw2, "d_shared": d_shared, "fwd": fwd}


# ---------------------------------------------------------------------------
# MXFP8 backward (Composer 2 Technical Report, §6.1 "Kernels": the MoE backward runs in
# MXFP8, E4M3 values with one E8M0 scale per block of 32; Figure 10: the layer is trained
# as one grouped-GEMM flow).  The page fixes the format, not the quantisation axes or
# the scale rule; the readings here:
#   * every backward GEMM takes both operands in MXFP8 blocked along that GEMM's own
#     reduction dimension, quantised from the exact value of the operand;
#   * the scale of a block is the smallest power of two X with amax / X <= 448 (no
#     element saturates), elements round to the nearest E4M3 value, ties to the even
#     code; an all-zero block has X = 2^-127 and zeros;
#   * the forward's h is quantised per row along I before the second GEMM (the MXFP8
#     forward), so hq is what the forward multiplied and what dW2 multiplies;
#   * data gradients (dh = d_out W2, dx = da W1 + dg W3) reduce over d or I: their
#     activation operands are quantised per row (token-local) and their weight operands
#     are the weights requantised along the other axis;
#   * weight gradients reduce over the expert's rows: both operands are quantised along
#     the rows in blocks of 32 starting at the expert's first row, the last block padded
#     with zeros.
# Everything else (products, sums, SwiGLU and its derivative) is exact float64.
# ---------------------------------------------------------------------------
def mx_quantize(v, axis: int = -1, block: int = 32) -> np.ndarray:
    """MXFP8 values of exact ``v`` blocked along ``axis`` (its length a multiple of
    ``block``): per block X = the smallest power of two with amax / X <= 448, clamped to
    2^-127 .. 2^127, elements X * E4M3_RNE(v / X).  Returns float64 values."""
    v = np.moveaxis(f64(v), axis, -1)
    K = v.shape[-1]
    assert K % block == 0
    b = v.reshape(v.shape[:-1] + (K // block, block))
    amax = np.abs(b).max(axis=-1)
    _, ex = np.frexp(amax)                       # amax = m 2^ex, m in [0.5, 1)
    e = ex.astype(np.int64) - 1 - 8              # floor(log2 amax) - 8
    e = np.where(np.ldexp(amax, -e) > 448.0, e + 1, e)
    e = np.where(amax == 0, -127, np.clip(e, -127, 127))
    q = np.ldexp(b, -e[..., None])               # exact: a power-of-two scaling
    idx, neg = _rne_codes(q, E4M3_TABLE[:127])   # magnitudes 0 .. 448 ascend with the code
    vals = np.where(neg, -1.0, 1.0) * E4M3_TABLE[idx]
    out = np.ldexp(vals, e[..., None]).reshape(v.shape)
    return np.moveaxis(out, -1, axis)


def _no_quant(v, axis: int = -1) -> np.ndarray:
    return f64(v)


def expert_forward_mxfp8(x_rows, w1, w3, w2, quant=mx_quantize):
    """One expert of the MXFP8 layer: a = x W1, g = x W3, hq = MX_I(silu(a) g) (per row),
    out = hq W2.  Returns (a, g, hq, out)."""
    xr = f64(x_rows)
    a = xr @ f64(w1).T
    g = xr @ f64(w3).T
    hq = quant(silu(a) * g, 1)
    return a, g, hq, hq @ f64(w2).T


def layer_mxfp8(x, w_gate, bias, experts, shared, k: int, ids_in=None, weights_in=None,
                quant=mx_quantize):
    """The MXFP8 layer's forward with h requantised to MXFP8 per row before the down
    projection (the MoE activations travel as E4M3 values with one E8M0 scale per 32:
    Composer 2 Technical Report, §6.1 "Kernels"; the scale rule is ``mx_quantize``'s):
    routing and dispatch as in ``layer``, each expert (and the shared one) through
    ``expert_forward_mxfp8``, the same combine.  Exact float64 otherwise."""
    xf = f64(x)
    T, d = xf.shape
    if ids_in is None:
        ids, w, logits = route(xf, w_gate, bias, k)
    else:
        ids, w, logits = route_replay(xf, w_gate, bias, ids_in, weights_in)
    E = logits.shape[1]
    offsets, perm, row_of = dispatch(ids, E)
    rows = np.zeros((T * k, d), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows[lo:hi] = expert_forward_mxfp8(xf[perm[lo:hi] // k], *experts[e], quant=quant)[3]
    y = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        for r in range(k):
            y[t] += w[t, r] * rows[row_of[t * k + r]]
    if shared is not None:
        y += expert_forward_mxfp8(xf, *shared, quant=quant)[3]
    return {"y": y, "ids": ids, "weights": w, "logits": logits,
            "offsets": offsets, "perm": perm, "row_of": row_of, "rows": rows}


def expert_forward_nvfp4(x_rows, w1, w3, w2):
    """One expert of the NVFP4 forward (``expert_ffn_nvfp4``), keeping what its MXFP8
    backward takes: (xq, a, g, hq, out, (W1, W3, W2)) with xq the rows quantized to NVFP4
    per row, a = xq W1, g = xq W3, hq = NVFP4(bf16(silu(a) g)) per row, out = hq W2, and
    the weights' exact values."""
    W1, W3, W2 = (nvfp4_dequant(*w) for w in (w1, w3, w2))
    xq = nvfp4_dequant(*nvfp4_quantize(np.asarray(x_rows, dtype=np.float32)))
    a = xq @ W1.T
    g = xq @ W3.T
    hq = nvfp4_dequant(*nvfp4_quantize(bf16_rne(silu(a) * g).astype(np.float32)))
    return xq, a, g, hq, hq @ W2.T, (W1, W3, W2)


def expert_backward_mxfp8(x_rows, a, g, hq, d_out_rows, w1, w3, w2, quant=mx_quantize):
    """The MXFP8 backward of one expert over its rows (readings above): returns (dx rows,
    dW1, dW3, dW2, dL/dh rows)."""
    xr = f64(x_rows)
    do = f64(d_out_rows)
    n = xr.shape[0]
    pad = (-n) % 32

    def rows(m):          # quantised along the rows, zero-padded to whole blocks
        mp = np.concatenate([m, np.zeros((pad, m.shape[1]))]) if pad else m
        return quant(mp, 0)[:n]

    dh = quant(do, 1) @ quant(w2, 0)
    da = dh * g * silu_grad(a)
    dg = dh * silu(a)
    dx = quant(da, 1) @ quant(w1, 0) + quant(dg, 1) @ quant(w3, 0)
    xq = rows(xr)
    return dx, rows(da).T @ xq, rows(dg).T @ xq, rows(do).T @ rows(hq), dh


def layer_backward_mxfp8(x, w_gate, bias, experts, shared, k: int, dy, ids_in=None,
                         weights_in=None, quant=mx_quantize, grad_round=None, forward="mxfp8"):
    """Gradients of L = <dy, y> through the MXFP8 layer, under the readings above.

    Same arguments and result keys as ``layer_backward`` (the inputs are the exact
    dequantised values), plus "y" (the forward with hq), "dh_rows" (dL/dh of every
    dispatched row, then the shared rows) and "hq_rows".  The gradient of each
    dispatched row's expert output, w_tr dy_t, is rounded to the layer's gradient type,
    bf16 (``grad_round``, default ``bf16_rne``), before it enters the expert backward.
    ``quant(v, axis)`` is the quantiser; an identity quantiser and rounding turn this
    into the exact chain rule of the unquantised layer (``layer_backward``).
    With forward="nvfp4" the layer's forward is the NVFP4 one (``layer_nvfp4``: experts
    and shared given as NVFP4 triples, x bf16): its backward is the same MXFP8 backward
    on the forward's operands as that forward quantized them (xq, the weights' NVFP4
    values, hq; Composer 2 Technical Report, §6.1 "Kernels": NVFP4 forward, MXFP8
    backward).
    """
    nv = forward == "nvfp4"
    if grad_round is None:
        grad_round = bf16_rne
    xf = f64(x)
    dyf = f64(dy)
    T, d = xf.shape
    if ids_in is None:
        ids, w, logits = route(xf, w_gate, bias, k)
    else:
        ids, w, logits = route_replay(xf, w_gate, bias, ids_in, weights_in)
    E = logits.shape[1]
    offsets, perm, row_of = dispatch(ids, E)
    I = f64(experts[0][0]).shape[0] if E and not nv else 0
    rows_out = np.zeros((T * k, d))
    saved = {}

    def fwd(xr, ws):
        if nv:
            return expert_forward_nvfp4(xr, *ws)
        a, g, hq, o = expert_forward_mxfp8(xr, *ws, quant=quant)
        return xr, a, g, hq, o, ws

    if nv and E:
        I = nvfp4_dequant(*experts[0][0]).shape[0]
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        xq, a, g, hq, o, wv = fwd(xf[perm[lo:hi] // k], experts[e])
        rows_out[lo:hi] = o
        saved[e] = (xq, a, g, hq, wv)
    y = np.zeros((T, d))
    for t in range(T):
        for r in range(k):
            y[t] += w[t, r] * rows_out[row_of[t * k + r]]
    if shared is not None:
        sxq, sa, sg, shq, so, swv = fwd(xf, shared)
        y += so
    d_weights = np.empty((T, k))
    d_rows = np.empty_like(rows_out)
    for t in range(T):
        for r in range(k):
            j = row_of[t * k + r]
            d_weights[t, r] = float(dyf[t] @ rows_out[j])
            d_rows[j] = grad_round(w[t, r] * dyf[t])
    dx = np.zeros((T, d))
    dw1, dw3, dw2 = {}, {}, {}
    dh_rows = np.zeros((T * k + (T if shared is not None else 0), I))
    hq_rows = np.zeros_like(dh_rows)
    for e, (xq, a, g, hq, wv) in saved.items():
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        toks = perm[lo:hi] // k
        gx, dw1[e], dw3[e], dw2[e], dh_rows[lo:hi] = expert_backward_mxfp8(
            xq, a, g, hq, d_rows[lo:hi], *wv, quant=quant)
        hq_rows[lo:hi] = hq
        np.add.at(dx, toks, gx)
    d_shared = None
    if shared is not None:
        gx, s1, s3, s2, dh_rows[T * k:] = expert_backward_mxfp8(sxq, sa, sg, shq, dyf, *swv, quant=quant)
        hq_rows[T * k:] = shq
        dx += gx
        d_shared = (s1, s3, s2)
    d_w_gate = np.zeros((d, E))
    d_bias = None if bias is None else np.zeros(E)
    if weights_in is None:
        dl = softmax_pick_grad(w, d_weights)
        wg = f64(w_gate)
        for t in range(T):
            for r in range(k):
                e = int(ids[t, r])
                dx[t] += dl[t, r] * wg[:, e]
                d_w_gate[:, e] += dl[t, r] * xf[t]
                if d_bias is not None:
                    d_bias[e] += dl[t, r]
    return {"dx": dx, "d_weights": d_weights, "d_w_gate": d_w_gate, "d_bias": d_bias,
            "dw1": dw1, "dw3": dw3, "dw2": dw2, "d_shared": d_shared, "y": y,
            "dh_rows": dh_rows, "hq_rows": hq_rows, "ids": ids, "weights": w,
            "offsets": offsets, "perm": perm, "row_of": row_of}


# ---------------------------------------------------------------------------
# NVFP4 (the forward-pass format of Composer 2 Technical Report, §6.1 "Kernels": FP4
# E2M1 values, one FP8 E4M3 scale per block of 16, one FP32 scale per token; the
# quantization uses IEEE division)
# ---------------------------------------------------------------------------
E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_value(code: int) -> float:
    """FP4 E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is
    the subnormal 0.5 m."""
    v = float(E2M1_MAGS[code & 7])
    return -v if code & 8 else v


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def _rne_codes(x, mags):
    """Codes (sign << k | magnitude index) of the nearest value on a non-negative grid
    `mags` (ascending, index = code magnitude bits), ties to the even index, saturating
    at the largest magnitude.  x: float values (exact)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), mags[-1])
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, len(mags) - 1)
    lo = np.clip(hi - 1, 0, len(mags) - 1)
    dlo, dhi = a - mags[lo], mags[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    return idx, np.signbit(x)


def e2m1_rne_codes(x) -> np.ndarray:
    """Nearest E2M1 code, ties to even, saturating at 6 (the sign kept, -0 -> 8)."""
    idx, neg = _rne_codes(x, E2M1_MAGS)
    return (idx + np.where(neg, 8, 0)).astype(np.uint8)


def e4m3_rne_codes(x) -> np.ndarray:
    """Nearest OCP E4M3 code, ties to even, saturating at 448 (non-negative inputs)."""
    mags = E4M3_TABLE[:127]            # codes 0x00..0x7E ascend in value; 0x7F is NaN
    idx, neg = _rne_codes(x, mags)
    assert not np.any(neg & (np.abs(np.asarray(x, dtype=np.float64)) > 0))
    return idx.astype(np.uint8)


def nvfp4_quantize(v):
    """Rows of v (exact fp32 values, K % 16 == 0) -> (codes [R, K] 0..15, block scale
    codes [R, K/16] E4M3, row scales [R] fp32).  Per row: s = amax / 2688 (6 * 448, the
    largest E2M1 times the largest E4M3); per block of 16: S = E4M3_RNE((bamax / s) / 6);
    per element: E2M1_RNE(v / (S s)).  Every step is one IEEE fp32 operation (division
    or product) rounded to nearest even, as numpy's float32 arithmetic is; a zero row
    gets s = 0 and zero codes, a zero block scale gives zero codes."""
    v = np.asarray(v, dtype=np.float32)
    R, K = v.shape
    assert K % 16 == 0
    blocks = v.reshape(R, K // 16, 16)
    amax = np.abs(v).max(axis=1) if K else np.zeros(R, np.float32)
    live = amax > 0
    s = np.zeros(R, np.float32)
    s[live] = amax[live] / np.float32(2688.0)
    bamax = np.abs(blocks).max(axis=2)
    t = np.zeros_like(bamax)
    t[live] = bamax[live] / s[live, None]
    sb = e4m3_rne_codes(t / np.float32(6.0))
    sbv = E4M3_TABLE[sb].astype(np.float32)
    den = sbv * s[:, None]                 # fp32 product
    codes = np.zeros((R, K // 16, 16), dtype=np.uint8)
    nz = den > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        q = blocks / den[..., None]        # fp32 division
    codes[nz] = e2m1_rne_codes(q[nz])
    return codes.reshape(R, K), sb, s


def nvfp4_dequant(codes, block_scales, row_scales) -> np.ndarray:
    """Exact values E2M1(code) * E4M3(block scale) * row scale, in float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    sb = E4M3_TABLE[np.asarray(block_scales, dtype=np.uint8)]
    return (E2M1_TABLE[codes] * np.repeat(sb, 16, axis=1)) * f64(row_scales)[:, None]


def bf16_rne(v) -> np.ndarray:
    """float64 -> float32 (nearest, ties to even) -> bf16 (nearest, ties to even), returned
    as float64: the bf16 rounding of the value's fp32 rounding, as for an h computed in fp32."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)   # fp64 -> fp32 RNE
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def expert_ffn_nvfp4(x_rows, w1, w3, w2) -> np.ndarray:
    """SwiGLU expert in the NVFP4 forward: the rows quantized per row (token), weights
    given as NVFP4 triples (codes, block scales, row scales) per matrix, h rounded to
    bf16 and quantized per row before the second GEMM; products exact in float64."""
    W1, W3, W2 = (nvfp4_dequant(*w) for w in (w1, w3, w2))
    xq = nvfp4_dequant(*nvfp4_quantize(np.asarray(x_rows, dtype=np.float32)))
    h = bf16_rne(silu(xq @ W1.T) * (xq @ W3.T))
    hq = nvfp4_dequant(*nvfp4_quantize(h.astype(np.float32)))
    return hq @ W2.T


def layer_nvfp4(x, w_gate, bias, experts, shared, k: int, ids_in=None, weights_in=None):
    """The layer forward with NVFP4 experts: routing on the bf16 x as in ``layer``, each
    expert (and the shared one) through ``expert_ffn_nvfp4``, the same combine."""
    xf = f64(x)
    T, d = xf.shape
    if ids_in is None:
        ids, w, logits = route(xf, w_gate, bias, k)
    else:
        ids, w, logits = route_replay(xf, w_gate, bias, ids_in, weights_in)
    E = logits.shape[1]
    offsets, perm, row_of = dispatch(ids, E)
    rows = np.zeros((T * k, d), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows[lo:hi] = expert_ffn_nvfp4(xf[perm[lo:hi] // k], *experts[e])
    y = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        for r in range(k):
            y[t] += w[t, r] * rows[row_of[t * k + r]]
    if shared is not None:
        y += expert_ffn_nvfp4(xf, *shared)
    return {"y": y, "ids": ids, "weights": w, "logits": logits,
            "offsets": offsets, "perm": perm, "row_of": row_of, "rows": rows}
