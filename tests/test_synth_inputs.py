"""The seeded input generator: MXFP8 encoder against the oracle's decoder, replay
draws, determinism and shapes (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.inputs import _e4m3_rne_codes

FINITE = [c for c in range(256) if not math.isnan(oracle.E4M3_TABLE[c])]


def _nearest_even_code(v):
    """Brute force: the finite E4M3 code nearest to v; ties go to the even mantissa."""
    best = None
    for c in FINITE:
        dist = abs(oracle.E4M3_TABLE[c] - v)
        key = (dist, c & 1, c & 0x80 if v >= 0 else (~c) & 0x80)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_e4m3_rounding_matches_brute_force():
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(300) * 30) + list(rng.standard_normal(100) * 0.01)
    pos = sorted(set(oracle.E4M3_TABLE[1:0x7F].tolist()))
    mids = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])]      # exact midpoints -> ties
    vals += mids + [-m for m in mids] + [448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -11, 0.0]
    q = torch.tensor(vals, dtype=torch.float64).clamp(-448, 448).to(torch.float32)
    codes = _e4m3_rne_codes(q).numpy()
    for v, c in zip(q.tolist(), codes.tolist()):
        want = _nearest_even_code(v)
        assert oracle.E4M3_TABLE[c] == oracle.E4M3_TABLE[want], (v, c, want)


def test_mx_quantize_scale_rule_and_round_trip():
    rng = np.random.default_rng(1)
    v = torch.from_numpy((rng.standard_normal((6, 128)) * np.array([1e-3, 1, 30, 1e4, 2.0 ** -100, 1])[:, None])
                         .astype(np.float32))
    v[5, 32:64] = 0.0                       # an all-zero block
    codes, scales = synth.mxfp8_quantize(v)
    amax = v.abs().reshape(6, 4, 32).amax(-1).double()
    for i in range(6):
        for b in range(4):
            if amax[i, b] == 0:
                assert scales[i, b] == 0
                assert torch.all(codes[i, 32 * b:32 * b + 32] == 0)
            else:
                assert int(scales[i, b]) - 127 == math.floor(math.log2(amax[i, b])) - 8
    deq = oracle.mx_dequant(codes.numpy(), scales.numpy())
    # in the scaled domain q = v / X the error is half an E4M3 ulp of q, or the
    # clamp to 448 when |q| lies in (448, 512)
    X = np.repeat(2.0 ** (scales.numpy().astype(np.float64) - 127), 32, axis=1)
    q = np.abs(v.double().numpy()) / X
    with np.errstate(divide="ignore"):
        ulp = np.where(q < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 3))
    bound = np.maximum(ulp / 2, q - 448.0) * X
    err = np.abs(deq - v.double().numpy())
    assert np.all(err <= bound)
    # already-representable values come back exactly
    codes2, scales2 = synth.mxfp8_quantize(torch.from_numpy(deq.astype(np.float32)))
    assert np.array_equal(oracle.mx_dequant(codes2.numpy(), scales2.numpy()), deq)


def test_zipf_replay_ids_and_dirichlet_weights():
    rng = np.random.Generator(np.random.PCG64(2))
    ids = synth.zipf_replay_ids(4096, 384, 8, 1.2, rng)
    w = synth.dirichlet_weights(4096, 8, rng)
    assert ids.dtype == np.int32 and ids.shape == (4096, 8)
    assert ids.min() >= 0 and ids.max() < 384
    assert all(len(set(r)) == 8 for r in ids.tolist())
    counts = np.bincount(ids.ravel(), minlength=384)
    assert counts[0] == counts.max() and counts[0] > 10 * np.median(counts)
    assert w.dtype == np.float32 and np.all(w > 0)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)


@pytest.mark.parametrize("name", ["tiny_fp32_t32"])
def test_make_layer_inputs_shapes_and_determinism(name):
    wl = synth.WORKLOADS[name]
    a = synth.make_layer_inputs(wl)
    b = synth.make_layer_inputs(wl)
    assert torch.equal(a["x"], b["x"]) and torch.equal(a["w2"], b["w2"])
    assert a["x"].shape == (wl.T, wl.d) and a["w_gate"].shape == (wl.d, wl.E)
    assert a["w1"].shape == (wl.E, wl.inter, wl.d) and a["w2"].shape == (wl.E, wl.d, wl.inter)
    assert a["x"].dtype == torch.float32
    # N(0, 1/fan_in): sample std close to 1/sqrt(fan_in)
    assert abs(a["w2"].std().item() * math.sqrt(wl.inter) - 1) < 0.02
    assert abs(a["w1"].std().item() * math.sqrt(wl.d) - 1) < 0.02


def test_small_bf16_mxfp8_replay_variants():
    base = synth.WORKLOADS["bf16_t4096"].with_(T=16, d=64, inter=32, E=12, k=3)
    a = synth.make_layer_inputs(base)
    assert a["x"].dtype == torch.bfloat16 and a["shared"]["w2"].shape == (64, 32)
    m = synth.make_layer_inputs(base.with_(dtype="mxfp8", bias=True))
    assert m["x"].dtype == torch.uint8 and m["x_scale"].shape == (16, 2)
    assert m["w2_scale"].shape == (12, 64, 1) and m["bias"].shape == (12,)
    r = synth.make_layer_inputs(base.with_(routing="replay"))
    assert r["ids_in"].shape == (16, 3) and r["weights_in"].dtype == torch.float32


def _mx_quantize_with_ldexp(v):
    """The encoder as first written (scaling by torch.ldexp), kept to show the
    power-of-two multiply that replaced it gives the same codes and scales."""
    shp = v.shape
    blocks = v.to(torch.float32).reshape(*shp[:-1], shp[-1] // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)
    se = (ex.to(torch.int64) - 1) - 8
    se = torch.where(amax == 0, torch.full_like(se, -127), se).clamp(-127, 127)
    q = torch.ldexp(blocks.to(torch.float64), (-se).unsqueeze(-1).to(torch.float64))
    q = q.clamp(-448.0, 448.0).to(torch.float32)
    return _e4m3_rne_codes(q).reshape(shp), (se + 127).to(torch.uint8)


def test_mx_quantize_equals_ldexp_form():
    rng = np.random.default_rng(3)
    rows = []
    for lg in range(-149, 128, 3):                      # every fp32 binade, subnormals included
        rows.append(rng.standard_normal(64) * 2.0 ** lg)
    v = np.concatenate([np.clip(np.stack(rows), -3.4e38, 3.4e38),
                        rng.standard_normal((64, 64))]).astype(np.float32)
    v[3, :32] = 0.0
    v[4, 5] = np.float32(3.4028235e38)
    v[5, 7] = -np.float32(1.4e-45)
    t = torch.from_numpy(v)
    c1, s1 = synth.mxfp8_quantize(t)
    c0, s0 = _mx_quantize_with_ldexp(t)
    assert torch.equal(c1, c0) and torch.equal(s1, s0)
    assert int(s1.min()) == 0 and int(s1.max()) == 127 + 119   # both ends of the E8M0 range met


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8", "nvfp4", "f32"])
def test_chunked_storage_equals_per_matrix_storage(dtype):
    """Expert weights are stored (rounded or quantised) 16 experts at a time; the
    result must equal storing each drawn matrix on its own, in the recipe's order."""
    from synth.inputs import _draw_gate, _store
    wl = synth.Workload("chunk", T=8, d=64, inter=32, E=37, k=2, shared=True, bias=True,
                        dtype=dtype, seed=11)
    got = synth.make_layer_inputs(wl)
    _, randn = _draw_gate(wl, "cpu", None)
    for e in list(range(wl.E)) + ["shared"]:
        for name, shape, fan in (("w1", (32, 64), 64), ("w3", (32, 64), 64), ("w2", (64, 32), 32)):
            st = _store(randn(*shape, std=1.0 / math.sqrt(fan)), dtype)
            src = got["shared"] if e == "shared" else {kk: v[e] for kk, v in got.items()
                                                        if kk[:2] in ("w1", "w3", "w2") and v is not None}
            assert torch.equal(src[name], st[0]), (e, name)
            if st[1] is not None:
                assert torch.equal(src[name + "_scale"], st[1])
            if len(st) > 2:
                assert torch.equal(src[name + "_rscale"], st[2])
