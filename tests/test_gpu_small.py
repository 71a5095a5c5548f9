"""GPU parity at sizes the oracle finishes in seconds: every token, element by element.

Routing ids and dispatch are compared bit-exactly, weights to 2e-6, the layer output
normwise to the dtype's bar; MXFP8 layers also against the oracle that requantises h
as the library does, to a relative Frobenius error of 6e-3.  Shapes span several GEMM tiles, ragged tails, one-token
batches, k = 1 and k = E, exact and near ties, zero inputs, the shared expert and the
gate bias.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parity_gate_gemm_amd as pg
import synth
from _gpu_common import (TOL, check_dispatch_properties, compare_rows, compare_rows_hq, host,
                         oracle_for_rows, run_layer, say, to_device)

pytestmark = pytest.mark.gpu


def _inputs(wl):
    return to_device(synth.make_layer_inputs(wl, device="cpu"))


def test_tiny_fp32_workload():
    wl = synth.WORKLOADS["tiny_fp32_t32"]
    say("case tiny_fp32_t32 seed 0")
    inp = _inputs(wl)
    res = run_layer(inp, wl.k)
    ref = oracle_for_rows(inp, np.arange(wl.T), wl.k)
    err = compare_rows(res, ref, np.arange(wl.T), "f32")
    assert np.array_equal(res["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(res["perm"].cpu().numpy(), ref["perm"])
    assert np.array_equal(res["row_of"].cpu().numpy(), ref["row_of"])
    say(f"  tiny fp32 normwise err {err:.3e}")
    assert err < 1e-5          # fp32 end to end: far inside the 2e-2 bar


def test_tiny_fp32_workload_determinism_permutation_single_tokens():
    wl = synth.WORKLOADS["tiny_fp32_t32"]
    say("case tiny_fp32_t32 determinism, permutation, single tokens")
    inp = _inputs(wl)
    base = run_layer(inp, wl.k)
    for _ in range(9):
        r = run_layer(inp, wl.k)
        assert torch.equal(r["y"], base["y"]) and torch.equal(r["ids"], base["ids"])
    p = torch.randperm(wl.T, generator=torch.Generator().manual_seed(0)).cuda()
    rp = run_layer(dict(inp, x=inp["x"][p].contiguous()), wl.k)
    assert torch.equal(rp["ids"], base["ids"][p])
    assert torch.equal(rp["weights"], base["weights"][p])
    assert torch.equal(rp["y"], base["y"][p])
    for t in range(wl.T):
        r1 = run_layer(dict(inp, x=inp["x"][t:t + 1].contiguous()), wl.k)
        assert torch.equal(r1["ids"][0], base["ids"][t])
        assert torch.equal(r1["weights"][0], base["weights"][t])
        assert torch.equal(r1["y"][0], base["y"][t])


SMALL = [
    # T, d, I, E, k, shared, bias, dtype
    (1, 128, 64, 16, 2, False, False, "bf16"),
    (37, 128, 64, 16, 4, True, False, "bf16"),
    (300, 256, 128, 4, 2, True, True, "bf16"),     # 150 rows/expert: 2 M-tiles, ragged
    (200, 128, 64, 384, 8, True, False, "bf16"),
    (64, 128, 64, 8, 8, False, True, "bf16"),      # k == E
    (129, 128, 64, 3, 1, False, False, "bf16"),    # k == 1, one expert gets >128 rows
    (200, 128, 128, 16, 4, True, True, "mxfp8"),
    (300, 256, 256, 4, 2, True, False, "mxfp8"),   # 150 rows/expert: 2 row tiles, ragged
    (1, 128, 128, 384, 8, False, True, "mxfp8"),
    # d and I multiples of 512: the MXFP8 GEMMs run on the LDS-ring tiles, 256 rows where the
    # experts average more than 128 routed rows, else 128 rows over three stages
    (700, 1024, 512, 16, 4, True, True, "mxfp8"),   # 175 rows/expert (1 ragged tile); shared 3 tiles
    (1500, 512, 512, 4, 2, False, False, "mxfp8"),  # 750 rows/expert: 3 row tiles, ragged
    (300, 512, 512, 8, 2, True, True, "mxfp8"),     # 128-row tiles: 75 rows/expert, skewed by the bias
    (100, 1024, 512, 32, 4, False, False, "mxfp8"), # 128-row tiles: ~12 rows/expert, one partial tile
    (50, 64, 32, 16, 3, True, True, "f32"),
    (5, 96, 40, 1024, 32, True, False, "f32"),     # largest E and k
]


@pytest.mark.parametrize("T,d,I,E,k,shared,bias,dtype", SMALL)
def test_small_layers(T, d, I, E, k, shared, bias, dtype):
    wl = synth.Workload("small", T=T, d=d, inter=I, E=E, k=k, shared=shared, bias=bias,
                        dtype=dtype, seed=100 + T + E)
    say(f"case small T={T} d={d} I={I} E={E} k={k} shared={shared} bias={bias} {dtype}")
    inp = _inputs(wl)
    res = run_layer(inp, k)
    ref = oracle_for_rows(inp, np.arange(T), k)
    err = compare_rows(res, ref, np.arange(T), dtype)
    assert np.array_equal(res["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(res["perm"].cpu().numpy(), ref["perm"])
    assert np.array_equal(res["row_of"].cpu().numpy(), ref["row_of"])
    say(f"  normwise err {err:.3e}")
    if dtype == "mxfp8":
        compare_rows_hq(res, oracle_for_rows(inp, np.arange(T), k, layer=oracle.layer_mxfp8), np.arange(T))


def test_exact_and_near_ties_and_zero_tokens():
    """Exact ties (duplicated gate columns, all-zero tokens) and near ties below the
    fp64 GEMM's error bound must be decided exactly as on the exact logits."""
    T, d, I, E, k = 96, 128, 64, 24, 6
    wl = synth.Workload("ties", T=T, d=d, inter=I, E=E, k=k, shared=False, dtype="bf16", seed=7)
    inp = synth.make_layer_inputs(wl)
    wg = inp["w_gate"]
    wg[:, 2] *= 3.0                            # large columns: usually in the top k
    wg[:, 4] *= 2.5
    wg[:, 9] = wg[:, 2]                        # exact tie between experts 2 and 9
    wg[:, 17] = wg[:, 4]                       # 17 differs from 4 by one ulp in row 0 only
    wg[0, 17] = torch.nextafter(wg[0, 4], torch.tensor(float("inf")))
    x = inp["x"]
    x[0:4] = 0                                 # all logits zero: 24-way tie
    # a tiny first component makes l_17 - l_4 far smaller than the fp64 GEMM's error
    # bound (which scales with ||x||), so the certificate fails and the exact path decides
    x[4:12, 0] = 2.0 ** -20
    x[8:12, 0] = -(2.0 ** -20)
    inp = to_device(inp)
    say("case ties")
    res = run_layer(inp, k)
    ref = oracle_for_rows(inp, np.arange(T), k)
    compare_rows(res, ref, np.arange(T), "bf16")
    ids = res["ids"].cpu().numpy()
    assert np.array_equal(ids[0], np.arange(k))
    for t in range(T):
        row = list(ids[t])
        if 9 in row:
            assert 2 in row and row.index(2) < row.index(9)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "mxfp8"])
def test_near_ties_below_fp32_resolution(dtype):
    """Two large gate columns differing by a relative 2^-18: their logits differ by ~1e-5
    for every token, far below what a bf16 or fp32 gate resolves and far above the fp64
    gate's bound; ids must equal the exact-logit selection for every dtype."""
    T, d, I, E, k = 256, 256, 128, 32, 4
    wl = synth.Workload("refine", T=T, d=d, inter=I, E=E, k=k, dtype=dtype, seed=13)
    inp = synth.make_layer_inputs(wl)
    wg = inp["w_gate"]
    wg[:, 5] *= 4.0
    wg[:, 6] = (wg[:, 5].double() * (1.0 + 2.0 ** -18)).float()
    inp = to_device(inp)
    say(f"case near ties {dtype}")
    res = run_layer(inp, k)
    ref = oracle_for_rows(inp, np.arange(T), k)
    compare_rows(res, ref, np.arange(T), dtype)
    ids = res["ids"].cpu().numpy()
    both = [t for t in range(T) if 5 in ids[t] and 6 in ids[t]]
    assert len(both) > T // 4          # the pair is usually selected together


def test_replay_own_ids_equals_learned_bitwise():
    wl = synth.Workload("rep", T=150, d=128, inter=64, E=32, k=4, shared=True, bias=True,
                        dtype="bf16", seed=11)
    inp = _inputs(wl)
    say("case replay==learned small")
    learned = run_layer(inp, wl.k)
    inp2 = dict(inp, ids_in=learned["ids"].clone(), weights_in=None)
    rep = run_layer(inp2, wl.k, replay=True)
    assert torch.equal(rep["weights"], learned["weights"])
    assert torch.equal(rep["y"], learned["y"])
    inp3 = dict(inp, ids_in=learned["ids"].clone(), weights_in=learned["weights"].clone())
    rep2 = run_layer(inp3, wl.k, replay=True)
    assert torch.equal(rep2["y"], learned["y"])


def test_replay_zipf_dirichlet_small():
    wl = synth.Workload("zipf", T=300, d=128, inter=64, E=64, k=8, shared=True, dtype="bf16",
                        routing="replay", seed=2)
    inp = _inputs(wl)
    say("case replay zipf small")
    res = run_layer(inp, wl.k, replay=True)
    res["ids"] = inp["ids_in"]
    ref = oracle_for_rows(inp, np.arange(wl.T), wl.k, replay=True)
    err = compare_rows(res, ref, np.arange(wl.T), "bf16", replay=True)
    assert torch.equal(res["weights"], inp["weights_in"])      # verbatim
    off, perm, row_of = oracle.dispatch(inp["ids_in"].cpu().numpy(), wl.E)
    assert np.array_equal(res["offsets"].cpu().numpy(), off)
    assert np.array_equal(res["perm"].cpu().numpy(), perm)
    say(f"  normwise err {err:.3e}")


def test_dispatch_standalone_skewed_and_empty():
    rng = np.random.Generator(np.random.PCG64(5))
    for T, E, k in [(1, 5, 3), (1000, 384, 8), (4099, 16, 2), (3000, 1024, 32)]:
        say(f"case dispatch T={T} E={E} k={k}")
        ids = synth.zipf_replay_ids(T, E, k, 1.2, rng)
        dev = torch.from_numpy(ids).cuda()
        ws = pg.Workspace(T, 64, E, k, 64, pg.MOE_BF16)
        off, perm, row_of = pg.moe_dispatch(dev, E, ws)
        assert pg.moe_check(ws) == 0
        o2, p2, r2 = oracle.dispatch(ids, E)
        assert np.array_equal(off.cpu().numpy(), o2)
        assert np.array_equal(perm.cpu().numpy(), p2)
        assert np.array_equal(row_of.cpu().numpy(), r2)
        check_dispatch_properties(dev, off, perm, row_of, E)
    # empty batch: all offsets zero
    ws = pg.Workspace(0, 64, 16, 2, 64, pg.MOE_BF16)
    off, _, _ = pg.moe_dispatch(torch.empty(0, 2, dtype=torch.int32, device="cuda"), 16, ws)
    assert torch.all(off == 0)


def test_empty_batch_layer():
    wl = synth.Workload("empty", T=0, d=128, inter=64, E=16, k=2, shared=True, dtype="bf16", seed=1)
    inp = _inputs(wl)
    res = run_layer(inp, 2)
    assert res["y"].shape == (0, 128)


def test_bad_replay_ids_are_flagged_not_faulting():
    wl = synth.Workload("bad", T=40, d=128, inter=64, E=16, k=4, shared=False, dtype="bf16", seed=3)
    inp = _inputs(wl)
    ids = torch.arange(4, dtype=torch.int32, device="cuda").repeat(40, 1)
    for bad_val, where in [(16, (3, 2)), (-1, (0, 0)), (None, (7, 1))]:
        b = ids.clone()
        if bad_val is None:
            b[where] = b[where[0], 0]          # duplicate within the row
        else:
            b[where] = bad_val
        say(f"case bad ids {bad_val}")
        with pytest.raises(pg.MoeError) as ei:
            run_layer(dict(inp, ids_in=b, weights_in=None), 4, replay=True)
        assert ei.value.status == 4            # MOE_ERR_BAD_IDS


def test_nonfinite_input_is_flagged():
    wl = synth.Workload("nan", T=8, d=128, inter=64, E=16, k=2, shared=False, dtype="bf16", seed=4)
    inp = _inputs(wl)
    inp["x"][3, 5] = float("nan")
    with pytest.raises(pg.MoeError) as ei:
        run_layer(inp, 2)
    assert ei.value.status == 5                # MOE_ERR_NONFINITE


@pytest.mark.parametrize("dtype,d,I", [("bf16", 256, 128), ("mxfp8", 256, 128), ("mxfp8", 1024, 512),
                                       ("f32", 128, 64)])
def test_determinism_permutation_and_batch_invariance_small(dtype, d, I):
    wl = synth.Workload("inv", T=333, d=d, inter=I, E=64, k=8, shared=True, bias=True,
                        dtype=dtype, seed=21)
    inp = _inputs(wl)
    say("case invariance small")
    base = run_layer(inp, wl.k)
    for _ in range(9):
        assert torch.equal(run_layer(inp, wl.k)["y"], base["y"])
    p = torch.randperm(wl.T, generator=torch.Generator().manual_seed(0)).cuda()
    perm_in = dict(inp, x=inp["x"][p].contiguous())
    if inp["x_scale"] is not None:
        perm_in["x_scale"] = inp["x_scale"][p].contiguous()
    yp = run_layer(perm_in, wl.k)["y"]
    assert torch.equal(yp, base["y"][p])
    # a token alone gives the same bits as in the batch
    for t in (0, 17, 332):
        one = dict(inp, x=inp["x"][t:t + 1].contiguous())
        if inp["x_scale"] is not None:
            one["x_scale"] = inp["x_scale"][t:t + 1].contiguous()
        assert torch.equal(run_layer(one, wl.k)["y"][0], base["y"][t])


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_gate_k_split_matches_unsplit(dtype):
    """d = 1024 cuts every gate sum into 4 parts.  A batch of 8192 tokens x 64 experts
    runs the parts one after another in each workgroup; a single token runs them in 4
    workgroups and adds the partial sums afterwards.  Both must give the same bits."""
    wl = synth.Workload("split", T=8192, d=1024, inter=128, E=64, k=4, shared=False, bias=True,
                        dtype=dtype, seed=31)
    inp = synth.make_layer_inputs(wl, device="cuda")
    say(f"case gate K-split {dtype}")
    base = run_layer(inp, wl.k)
    for t in (0, 4097, 8191):
        one = dict(inp, x=inp["x"][t:t + 1].contiguous())
        if inp["x_scale"] is not None:
            one["x_scale"] = inp["x_scale"][t:t + 1].contiguous()
        r = run_layer(one, wl.k)
        assert torch.equal(r["ids"][0], base["ids"][t])
        assert torch.equal(r["weights"][0], base["weights"][t])
        assert torch.equal(r["y"][0], base["y"][t])
    rows = np.array([0, 4097, 8191])
    compare_rows(base, oracle_for_rows(inp, rows, wl.k), rows, dtype)


def test_mxfp8_h_requantisation_without_saturation():
    """A layer whose error against the oracle was 6.1e-2 when h blocks took the OCP
    suggested scale 2^(floor(log2 amax) - 8) (block maxima clamped to 448); with the
    smallest non-saturating power-of-two scale it is about 3e-2 (bar 6e-2)."""
    wl = synth.Workload("small", T=700, d=1024, inter=512, E=16, k=4, shared=True, bias=True,
                        dtype="mxfp8", seed=1016)
    say("case mxfp8 T=700 d=1024 I=512 E=16 k=4 seed 1016 (drawn on the GPU)")
    inp = synth.make_layer_inputs(wl, device="cuda")
    res = run_layer(inp, wl.k)
    rows = np.arange(wl.T)
    err = compare_rows(res, oracle_for_rows(inp, rows, wl.k), rows, "mxfp8")
    assert err <= 4.5e-2, err
    compare_rows_hq(res, oracle_for_rows(inp, rows, wl.k, layer=oracle.layer_mxfp8), rows)


def test_mxfp8_persistent_gemm2_several_tiles_per_workgroup():
    """An MXFP8 layer on the 256-row ring tiles whose down projection has 48 row tiles x
    16 column tiles = 768 tiles, three per workgroup of the persistent GEMM2 (one per CU):
    every workgroup finishes a tile's epilogue while the next tile's first loads are in
    flight.  Sampled rows against the oracle, the routing and dispatch of every token,
    bitwise repeats and one token alone (128-row tiles, one tile per workgroup) against
    its row in the batch."""
    from _gpu_common import check_routing_every_token, sample_rows
    wl = synth.Workload("pers", T=4096, d=4096, inter=512, E=8, k=2, shared=True, bias=True,
                        dtype="mxfp8", seed=77)
    say("case mxfp8 persistent GEMM2 T=4096 d=4096 I=512 E=8 k=2 shared bias")
    inp = synth.make_layer_inputs(wl, device="cuda")
    base = run_layer(inp, wl.k)
    check_routing_every_token(inp, base, wl.k, wl.E)
    rows = sample_rows(base["ids"].cpu().numpy(), base["offsets"].cpu().numpy(),
                       base["perm"].cpu().numpy(), wl.k, 256, True, 48, seed=5)
    compare_rows(base, oracle_for_rows(inp, rows, wl.k), rows, "mxfp8")
    compare_rows_hq(base, oracle_for_rows(inp, rows, wl.k, layer=oracle.layer_mxfp8), rows)
    for _ in range(3):
        assert torch.equal(run_layer(inp, wl.k)["y"], base["y"])
    for t in (0, 2049, 4095):
        one = dict(inp, x=inp["x"][t:t + 1].contiguous(), x_scale=inp["x_scale"][t:t + 1].contiguous())
        assert torch.equal(run_layer(one, wl.k)["y"][0], base["y"][t])
