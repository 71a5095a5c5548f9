"""Seeded synthetic layer inputs (shapes and distributions of the five workloads).

Draw recipe, fixed so a seed names one input set:
  * one ``torch.Generator`` on the drawing device, seeded with the workload seed;
  * draw order: x, gate weight, gate bias (if any), then for e = 0..E-1 the
    triple W1[e], W3[e], W2[e], then the shared expert's W1, W3, W2;
  * x ~ N(0, 1); every weight ~ N(0, 1/fan_in) with fan_in = d for the gate,
    W1 and W3 and fan_in = I for W2 (the second argument of N is a variance);
    the optional per-expert logit bias ~ N(0, 0.5);
  * draws are fp32, then stored as fp32, as bf16 (round to nearest even), or as
    OCP MXFP8 (E4M3 elements, one E8M0 scale per 32 consecutive elements of the
    contiguous dimension);
  * replayed routing (IDs, then weights) is drawn on the host from
    ``numpy.random.Generator(PCG64(seed))``.

Storage layout (row-major, the contiguous dimension last):
  x [T, d]; w_gate [d, E]; bias [E];
  w1, w3 [E, I, d] and w2 [E, d, I] -- each expert matrix is stored output-major
  (one contiguous input-length vector per output feature), so both grouped GEMMs
  read their weight operand along the reduction dimension;
  the shared expert's matrices have the same per-expert shapes.

The same seed drawn on a different device (CPU vs GPU generator) gives a
different, equally valid input set; a test always hands one drawn set to both
the oracle and the HIP path.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    inter: int
    E: int = 384
    k: int = 8
    shared: bool = False
    dtype: str = "bf16"          # "f32" | "bf16" | "mxfp8" | "nvfp4" (bf16 x, NVFP4 experts)
    routing: str = "learned"     # "learned" | "replay"
    bias: bool = False
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the benchmark brief, named by what they are.
WORKLOADS = {
    "tiny_fp32_t32": Workload("tiny_fp32_t32", T=32, d=128, inter=64, dtype="f32", seed=0),
    "bf16_t4096": Workload("bf16_t4096", T=4096, d=7168, inter=2048, shared=True,
                           dtype="bf16", seed=1),
    "replay_zipf_t4096": Workload("replay_zipf_t4096", T=4096, d=7168, inter=2048,
                                  shared=True, dtype="bf16", routing="replay", seed=2),
    "bf16_t128_stream": Workload("bf16_t128_stream", T=128, d=7168, inter=2048,
                                 dtype="bf16", seed=3),
    "mxfp8_t32768": Workload("mxfp8_t32768", T=32768, d=7168, inter=2048, shared=True,
                             dtype="mxfp8", bias=True, seed=4),
    # the MXFP8 layer at the training batch of the bf16 layer (the backward's workload)
    "mxfp8_t4096": Workload("mxfp8_t4096", T=4096, d=7168, inter=2048, shared=True,
                            dtype="mxfp8", bias=True, seed=6),
    # the bf16 T = 4096 layer with NVFP4 experts (the pages' forward format)
    "nvfp4_t4096": Workload("nvfp4_t4096", T=4096, d=7168, inter=2048, shared=True,
                            dtype="nvfp4", seed=5),
}


def bf16_round(t: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16, round to nearest even (torch's conversion)."""
    return t.to(torch.bfloat16)


# ---------------------------------------------------------------------------
# OCP MX v1.0 MXFP8 (E4M3 elements, E8M0 shared scale, block of 32)
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0
E4M3_EMAX = 8      # exponent of the largest normal E4M3 value (448 = 1.75 * 2^8)
MX_BLOCK = 32


def _e4m3_rne_codes(q: torch.Tensor) -> torch.Tensor:
    """fp32 values already clamped to [-448, 448] -> E4M3 codes, round to nearest even.

    Done with integer arithmetic on the fp32 bit pattern so the rounding rule is
    explicit (no reliance on a library cast's saturation/rounding behaviour).
    """
    q = q.to(torch.float32)
    sign = (q < 0) | ((q == 0) & (torch.signbit(q)))
    a = q.abs()
    bits = a.view(torch.int32).to(torch.int64)
    exp32 = (bits >> 23) & 0xFF            # biased fp32 exponent
    man32 = bits & 0x7FFFFF
    unb = exp32 - 127                       # unbiased exponent (for normals)
    # E4M3: normals have unbiased exponent -6..8, subnormals step 2^-9.
    # Number of fp32 mantissa bits to drop: normal -> 20; subnormal range -> more.
    is_norm8 = unb >= -6
    shift = torch.where(is_norm8, torch.full_like(unb, 20), 20 + (-6 - unb))
    shift = shift.clamp(max=62)
    full = torch.where(exp32 > 0, man32 | (1 << 23), man32)   # implicit bit
    # value = full * 2^(unb-23); target grid step is 2^(unb-23+shift)
    keep = full >> shift
    rem = full - (keep << shift)
    half = torch.where(shift > 0, torch.ones_like(shift) << (shift - 1), torch.zeros_like(shift))
    round_up = (rem > half) | ((rem == half) & (shift > 0) & ((keep & 1) == 1))
    keep = keep + round_up.to(torch.int64)
    # Re-express as E4M3 code: grid value = keep * 2^(unb-23+shift)
    # normal: keep in [8, 16] (16 = carry into next exponent)
    code = torch.zeros_like(keep)
    norm_e = unb + 7                        # biased E4M3 exponent for normals
    carry = is_norm8 & (keep == 16)
    e_fin = torch.where(carry, norm_e + 1, norm_e)
    m_fin = torch.where(carry, torch.zeros_like(keep), keep - 8)
    code_norm = (e_fin << 3) | m_fin
    # subnormal grid: value = keep * 2^-9 with keep in [0, 8]; keep == 8 is the
    # smallest normal (exponent field 1, mantissa 0) which the same formula gives.
    code_sub = keep  # exponent field 0 and mantissa keep (keep==8 -> 0b0001000)
    code = torch.where(is_norm8, code_norm, code_sub)
    code = torch.where(a == 0, torch.zeros_like(code), code)
    code = code | (sign.to(torch.int64) << 7)
    return code.to(torch.uint8)


def mxfp8_quantize(v: torch.Tensor):
    """Quantise fp32 ``v[..., K]`` (K % 32 == 0) to MXFP8 along the last dim.

    OCP MX v1.0: shared scale X = 2^(floor(log2(amax)) - emax_elem) with emax_elem = 8
    for E4M3, stored as E8M0 (biased by 127); elements = RNE_E4M3(v / X), clamped to
    +-448.  An all-zero block gets scale code 0 and zero elements.
    Returns (codes uint8 [..., K], scales uint8 [..., K/32]).
    """
    assert v.shape[-1] % MX_BLOCK == 0
    shp = v.shape
    blocks = v.to(torch.float32).reshape(*shp[:-1], shp[-1] // MX_BLOCK, MX_BLOCK)
    amax = blocks.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)               # amax = m * 2^ex, m in [0.5, 1)
    se = (ex.to(torch.int64) - 1) - E4M3_EMAX
    se = torch.where(amax == 0, torch.full_like(se, -127), se).clamp(-127, 127)
    # v / X = v * 2^-se, exact in float64: 2^-se (|se| <= 127) is built from its
    # exponent bits and the fp32 values times it neither overflow nor underflow.
    pow2 = ((1023 - se) << 52).view(torch.float64)
    q = blocks.to(torch.float64) * pow2.unsqueeze(-1)
    q = q.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float32)
    codes = _e4m3_rne_codes(q).reshape(shp)
    scales = (se + 127).to(torch.uint8)
    return codes, scales


E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)   # midpoints of 0, .5, 1, 1.5, 2, 3, 4, 6
NV_BLOCK = 16


def _e2m1_rne_codes(q: torch.Tensor) -> torch.Tensor:
    """fp32 values -> FP4 E2M1 codes (sign bit 3), nearest, ties to the even code,
    saturating at 6."""
    a = q.abs().clamp(max=6.0)
    mids = torch.tensor(E2M1_MIDS, dtype=torch.float32, device=q.device)
    idx = torch.bucketize(a, mids)                       # first midpoint >= a
    tie = (idx < len(E2M1_MIDS)) & (a == mids[idx.clamp(max=len(E2M1_MIDS) - 1)])
    idx = torch.where(tie & (idx % 2 == 1), idx + 1, idx)
    sign = torch.signbit(q).to(torch.int64)
    return (idx | (sign << 3)).to(torch.uint8)


def nvfp4_quantize(v: torch.Tensor):
    """Quantise fp32 ``v[..., K]`` (K % 16 == 0) to NVFP4 along the last dim: row scale
    s = amax / 2688 (fp32), block scale E4M3_RNE((bamax / s) / 6) per 16, elements
    E2M1_RNE(v / (S s)).  Returns (codes packed two per byte, element 2i in the low
    nibble [..., K/2] uint8, block scales [..., K/16] uint8 E4M3, row scales [...] fp32)."""
    assert v.shape[-1] % NV_BLOCK == 0
    shp = v.shape
    v = v.to(torch.float32)
    blocks = v.reshape(*shp[:-1], shp[-1] // NV_BLOCK, NV_BLOCK)
    amax = v.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / 2688.0, torch.zeros_like(amax))
    bamax = blocks.abs().amax(dim=-1)
    safe = torch.where(s > 0, s, torch.ones_like(s)).unsqueeze(-1)
    t = torch.where(s.unsqueeze(-1) > 0, bamax / safe, torch.zeros_like(bamax))
    sb = _e4m3_rne_codes((t / 6.0).clamp(max=E4M3_MAX))
    sbv = _e4m3_values(sb)
    den = sbv * s.unsqueeze(-1)
    q = blocks / torch.where(den > 0, den, torch.ones_like(den)).unsqueeze(-1)
    codes = torch.where(den.unsqueeze(-1) > 0, _e2m1_rne_codes(q), torch.zeros_like(q, dtype=torch.uint8))
    codes = codes.reshape(*shp[:-1], shp[-1])
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed.contiguous(), sb.contiguous(), s.contiguous()


def _e4m3_values(c: torch.Tensor) -> torch.Tensor:
    """E4M3 codes (non-negative, finite) -> fp32 values."""
    c = c.to(torch.int64)
    e, m = (c >> 3) & 15, c & 7
    sub = m.to(torch.float32) * 2.0 ** -9
    nor = (1.0 + m.to(torch.float32) / 8.0) * torch.pow(2.0, (e - 7).to(torch.float32))
    return torch.where(e == 0, sub, nor)


# ---------------------------------------------------------------------------
# Replayed routing for the router-replay workload
# ---------------------------------------------------------------------------
def zipf_replay_ids(T: int, E: int, k: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """[T, k] int32 expert IDs, distinct per row, drawn from a Zipf(s) popularity.

    Popularity rank r (1-based) maps to expert r-1, p_r proportional to r^-s.  Each
    row draws k experts without replacement by the Gumbel-top-k trick on log p;
    columns are in descending Gumbel key order.
    """
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    order = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return order.astype(np.int32)


def dirichlet_weights(T: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """[T, k] fp32 combine weights, Dirichlet(1, ..., 1) per row."""
    return rng.dirichlet(np.ones(k), size=T).astype(np.float32)


# ---------------------------------------------------------------------------
# Whole-layer inputs
# ---------------------------------------------------------------------------
def _store(v: torch.Tensor, dtype: str):
    if dtype == "f32":
        return v.contiguous(), None
    if dtype == "bf16":
        return bf16_round(v).contiguous(), None
    if dtype == "mxfp8":
        return mxfp8_quantize(v)
    if dtype == "nvfp4":
        return nvfp4_quantize(v)
    raise ValueError(dtype)


def _draw_gate(wl: Workload, device: str, draw_device: str | None):
    """The first draws of the recipe (x, gate weight, gate bias) and the generator's
    draw function, positioned for the expert weights."""
    dd = draw_device or device
    g = torch.Generator(device=dd)
    g.manual_seed(wl.seed)

    def randn(*shape, std=1.0):
        t = torch.randn(*shape, generator=g, device=dd, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t

    out = {}
    x, xs = _store(randn(wl.T, wl.d), "bf16" if wl.dtype == "nvfp4" else wl.dtype)   # NVFP4 layers take bf16 x
    out["x"], out["x_scale"] = x.to(device), (xs.to(device) if xs is not None else None)
    out["w_gate"] = randn(wl.d, wl.E, std=1.0 / math.sqrt(wl.d)).to(device)
    out["bias"] = randn(wl.E, std=math.sqrt(0.5)).to(device) if wl.bias else None
    return out, randn


def make_gate_inputs(wl: Workload, device: str = "cpu", draw_device: str | None = None):
    """Only the routing inputs of ``make_layer_inputs`` (x, x_scale, w_gate, bias),
    the same values for the same seed and draw device, without drawing the experts."""
    return _draw_gate(wl, device, draw_device)[0]


EXPERT_CHUNK = 16    # experts whose weights are stored (rounded / quantised) together


def make_layer_inputs(wl: Workload, device: str = "cpu", draw_device: str | None = None):
    """Draw one layer's inputs for workload ``wl`` (see module docstring for the recipe).

    Tensors are drawn on ``draw_device`` (default: ``device``) and returned on
    ``device``.  Returns a dict with keys
      x, x_scale, w_gate, bias, w1, w3, w2, w1_scale, w3_scale, w2_scale,
      shared (dict with the same weight keys, or None), ids_in, weights_in.
    ``*_scale`` are None unless the workload is MXFP8; ``ids_in``/``weights_in`` are
    None unless the workload replays routing.
    """
    out, randn = _draw_gate(wl, device, draw_device)
    T, d, I, E = wl.T, wl.d, wl.inter, wl.E

    elt = {"f32": torch.float32, "bf16": torch.bfloat16, "mxfp8": torch.uint8, "nvfp4": torch.uint8}[wl.dtype]
    pk = 2 if wl.dtype == "nvfp4" else 1      # NVFP4: two codes per byte

    def bank(n):
        t = {"w1": torch.empty(n, I, d // pk, dtype=elt, device=device),
             "w3": torch.empty(n, I, d // pk, dtype=elt, device=device),
             "w2": torch.empty(n, d, I // pk, dtype=elt, device=device)}
        if wl.dtype == "nvfp4":
            t["w1_scale"] = torch.empty(n, I, d // NV_BLOCK, dtype=torch.uint8, device=device)
            t["w3_scale"] = torch.empty(n, I, d // NV_BLOCK, dtype=torch.uint8, device=device)
            t["w2_scale"] = torch.empty(n, d, I // NV_BLOCK, dtype=torch.uint8, device=device)
            t["w1_rscale"] = torch.empty(n, I, dtype=torch.float32, device=device)
            t["w3_rscale"] = torch.empty(n, I, dtype=torch.float32, device=device)
            t["w2_rscale"] = torch.empty(n, d, dtype=torch.float32, device=device)
        elif wl.dtype == "mxfp8":
            t["w1_scale"] = torch.empty(n, I, d // MX_BLOCK, dtype=torch.uint8, device=device)
            t["w3_scale"] = torch.empty(n, I, d // MX_BLOCK, dtype=torch.uint8, device=device)
            t["w2_scale"] = torch.empty(n, d, I // MX_BLOCK, dtype=torch.uint8, device=device)
        else:
            t["w1_scale"] = t["w3_scale"] = t["w2_scale"] = None
        return t

    shapes = (("w1", (I, d), d), ("w3", (I, d), d), ("w2", (d, I), I))

    def fill(b, e0, n):
        """Experts e0 .. e0 + n - 1: drawn one matrix at a time in the recipe's order,
        then stored (rounded or quantised) together; every storage rule acts on rows of
        one matrix, so the result equals storing each matrix on its own."""
        stage = {name: torch.empty((n,) + shape, dtype=torch.float32, device=draw_dev)
                 for name, shape, _ in shapes}
        for i in range(n):
            for name, shape, fan in shapes:
                stage[name][i].copy_(randn(*shape, std=1.0 / math.sqrt(fan)))
        for name, _, _ in shapes:
            st = _store(stage[name], wl.dtype)
            b[name][e0:e0 + n].copy_(st[0])
            if st[1] is not None:
                b[name + "_scale"][e0:e0 + n].copy_(st[1])
            if len(st) > 2:
                b[name + "_rscale"][e0:e0 + n].copy_(st[2])
            del st
        del stage

    draw_dev = draw_device or device
    routed = bank(E)
    for e0 in range(0, E, EXPERT_CHUNK):
        fill(routed, e0, min(EXPERT_CHUNK, E - e0))
    out.update(routed)
    if wl.shared:
        sh = bank(1)
        fill(sh, 0, 1)
        out["shared"] = {kk: (vv[0] if vv is not None else None) for kk, vv in sh.items()}
    else:
        out["shared"] = None

    if wl.routing == "replay":
        rng = np.random.Generator(np.random.PCG64(wl.seed))
        ids = zipf_replay_ids(T, E, wl.k, 1.2, rng)
        wts = dirichlet_weights(T, wl.k, rng)
        out["ids_in"] = torch.from_numpy(ids).to(device)
        out["weights_in"] = torch.from_numpy(wts).to(device)
    else:
        out["ids_in"] = None
        out["weights_in"] = None
    return out
