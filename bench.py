#!/usr/bin/env python3
"""Benchmark of one MoE-layer forward on one MI355X.

A step is one pass of the whole hot path over one batch: gate GEMM + top-k +
softmax-renormalise (or router replay), counting-sort dispatch, grouped SwiGLU FFN
(W1/W3 GEMM with the SwiGLU epilogue, then the W2 GEMM) and the fixed-order
combine, all through the libmoe C ABI on the current stream.  Inputs are drawn
once, on the GPU, before timing and stay resident in HBM.

Prints one JSON line with tokens/s, per-stage HIP-event durations, the roofline of
the dominant kernel and the CPU oracle timed on a bounded token sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + MFMA util, 384-expert top-8 d=7168 T=4096 bf16"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
MXFP8_MFMA_PEAK_TFLOPS = 5000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bf16_t4096",
                    help="bf16_t4096 (default), replay_zipf_t4096, bf16_t128_stream, tiny_fp32_t32")
    ap.add_argument("--replay-filter", type=float, default=None, metavar="LOG_TAU",
                    help="replay workloads: route with the plausibility filter at ln tau = LOG_TAU "
                         "(the replayed ids are filtered and the weights come from the gate)")
    ap.add_argument("--backward", action="store_true",
                    help="bf16, MXFP8 and NVFP4 workloads: a step is the forward and the backward pass of the "
                         "layer (dL/dy drawn once, fp32 weight and gate gradients)")
    ap.add_argument("--cpu-sample", type=int, default=32,
                    help="tokens of the same batch the CPU oracle is timed on (0: skip)")
    ap.add_argument("--calibrate-copy", type=float, default=0.0, metavar="GIB",
                    help="only run a plain device-to-device copy of GIB GiB (three times), the "
                         "reference for scaling the FETCH_SIZE/WRITE_SIZE counters, and exit")
    return ap.parse_args()


def calibrate_copy(gib: float):
    import torch
    n = int(gib * (1 << 30))
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {n} bytes x3 (one copy kernel per iteration)")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU hot path only; --gpus must be 1 "
              "(the layer is not sharded across GPUs in this library).", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy > 0:
        calibrate_copy(args.calibrate_copy)
        return

    import numpy as np
    import torch

    import parity_gate_gemm_amd as pg
    import synth

    pg.lib()  # fail loudly if the HIP library is missing
    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_draw = time.perf_counter()
    inp = synth.make_layer_inputs(wl, device="cuda")
    torch.cuda.synchronize()
    t_draw = time.perf_counter() - t_draw

    T, d, E, k, I = wl.T, wl.d, wl.E, wl.k, wl.inter
    dt = {"f32": pg.MOE_F32, "bf16": pg.MOE_BF16, "mxfp8": pg.MOE_MXFP8, "nvfp4": pg.MOE_NVFP4}[wl.dtype]
    xdt = pg.MOE_BF16 if dt == pg.MOE_NVFP4 else dt     # NVFP4 layers: bf16 x, y, routing
    replay = wl.routing == "replay"
    filt = args.replay_filter
    if filt is not None and not replay:
        print("--replay-filter needs a replay workload (replay_zipf_t4096)", file=sys.stderr)
        sys.exit(2)
    has_shared = inp["shared"] is not None
    bwd = args.backward
    if bwd and wl.dtype not in ("bf16", "mxfp8", "nvfp4"):
        print("--backward runs the bf16, MXFP8 and NVFP4 workloads only", file=sys.stderr)
        sys.exit(2)
    mxb = bwd and wl.dtype in ("mxfp8", "nvfp4")     # the backward in MXFP8
    ws = pg.BackwardWorkspace(T, d, E, k, I, dt) if bwd else pg.Workspace(T, d, E, k, I, dt)
    x, wg, bias = inp["x"], inp["w_gate"], inp["bias"]
    # NVFP4 banks run K-blocked (packed once here, outside the timed region); the oracle
    # baseline reads the row-major form in `inp`
    run_inp = pg.nvfp4_pack_inputs(inp) if wl.dtype == "nvfp4" else inp
    routed = {n: run_inp.get(n) for n in ("w1", "w3", "w2") + pg._BANK_OPT}
    shared = run_inp["shared"]
    rows = T * k + (T if has_shared else 0)
    odt = torch.float32 if dt == pg.MOE_F32 else torch.bfloat16
    ids = inp["ids_in"] if replay and filt is None else torch.empty(T, k, dtype=torch.int32, device=dev)
    weights = torch.empty(T, k, dtype=torch.float32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    row_of = torch.empty(T * k, dtype=torch.int32, device=dev)
    out = torch.empty(rows, d, dtype=odt, device=dev)
    y = torch.empty(T, d, dtype=odt, device=dev)
    if bwd:
        gen = torch.Generator(device=dev)
        gen.manual_seed(wl.seed + 100)
        dy = torch.randn(T, d, generator=gen, device=dev).to(odt)
        d_out = torch.empty(rows, d, dtype=odt, device=dev)
        d_weights = torch.empty(T, k, dtype=torch.float32, device=dev)
        dx_rows = torch.empty(rows, d, dtype=torch.float32, device=dev)
        gshape = lambda b, n: b[n].shape[:-1] + ((d if n != "w2" else I),)  # noqa: E731  (NVFP4: packed codes)
        grads = {n: torch.empty(gshape(routed, n), dtype=torch.float32, device=dev) for n in ("w1", "w3", "w2")}
        sgrads = ({n: torch.empty(gshape(shared, n), dtype=torch.float32, device=dev) for n in ("w1", "w3", "w2")}
                  if has_shared else None)
        dx = torch.empty(T, d, dtype=torch.float32, device=dev)
        pre = torch.empty(rows, 2 * I, dtype=torch.float32, device=dev)
        gate_grad = not (replay and filt is None and inp["weights_in"] is not None)
        if mxb:   # the weights requantised for the backward: once per weight version, untimed
            tb_r = pg.moe_mxfp8_transpose_weights(routed)
            tb_s = pg.moe_mxfp8_transpose_weights(shared) if has_shared else None

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if filt is not None:
            pg.moe_route_replay_filtered(x, wg, bias, inp["ids_in"], filt, ws, x_scale=inp["x_scale"],
                                         ids_out=ids, weights_out=weights)
        elif replay:
            pg.moe_route_replay(x, wg, bias, ids, ws, weights_in=inp["weights_in"],
                                x_scale=inp["x_scale"], weights_out=weights)
        else:
            pg.moe_route(x, wg, bias, k, ws, x_scale=inp["x_scale"], ids=ids, weights=weights)
        if ev is not None:
            ev[1].record()
        pg.moe_dispatch(ids, E, ws, offsets=offsets, perm=perm, row_of=row_of)
        if ev is not None:
            ev[2].record()
        if bwd:   # training step: keep the pre-activations for the backward
            pg.moe_expert_ffn_gate_up_save(x, routed, shared, offsets, perm, k, ws, pre=pre,
                                           x_scale=inp["x_scale"])
        else:
            pg.moe_expert_ffn_gate_up(x, routed, shared, offsets, perm, k, ws, x_scale=inp["x_scale"])
        if ev is not None:
            ev[3].record()
        pg.moe_expert_ffn_down(dt, T, d, routed, shared, k, ws, out=out)
        if ev is not None:
            ev[4].record()
        pg.moe_combine(out, row_of, weights, T, has_shared, xdt, y=y)
        if ev is not None:
            ev[5].record()
        if not bwd:
            return
        pg.moe_combine_backward(dy, out, row_of, weights, T, has_shared, xdt, d_out=d_out, d_weights=d_weights)
        if ev is not None:
            ev[6].record()
        if mxb and wl.dtype == "nvfp4":
            pg.moe_expert_ffn_backward_nvfp4(x, routed, shared, tb_r, tb_s, offsets, perm, k, d_out, ws, pre,
                                             dx_rows=dx_rows, grads=grads, shared_grads=sgrads)
        elif mxb:
            pg.moe_expert_ffn_backward_mxfp8(x, inp["x_scale"], routed, shared, tb_r, tb_s, offsets, perm, k, d_out,
                                             ws, pre=pre, dx_rows=dx_rows, grads=grads, shared_grads=sgrads)
        else:
            pg.moe_expert_ffn_backward_data(x, routed, shared, offsets, perm, k, d_out, ws, dx_rows=dx_rows,
                                            pre=pre)
            if ev is not None:
                ev[7].record()
            pg.moe_expert_ffn_backward_weights(x, routed, shared, perm, k, d_out, ws, grads=grads,
                                               shared_grads=sgrads)
        if ev is not None:
            ev[8 - mxb].record()
        pg.moe_route_backward(x, wg, ids, weights, d_weights, offsets, perm, row_of, dx_rows, has_shared, ws,
                              gate_grad=gate_grad, bias_grad=bias is not None, dx=dx, x_scale=inp["x_scale"])
        if ev is not None:
            ev[9 - mxb].record()

    for _ in range(args.warmup):
        step()
    st = pg.moe_check(ws)
    if st != 0:
        raise pg.MoeError(st, "warmup")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range((9 if mxb else 10) if bwd else 6)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = pg.moe_check(ws)
    if st != 0:
        raise pg.MoeError(st, "timed steps")

    names = ["route", "dispatch", "ffn_gate_up", "ffn_down", "combine"]
    if mxb:
        names += ["combine_backward", "ffn_backward", "route_backward"]
    elif bwd:
        names += ["combine_backward", "ffn_backward_data", "ffn_backward_weights", "route_backward"]
    stage_ms = {n: float(np.mean([events[i][j].elapsed_time(events[i][j + 1])
                                  for i in range(args.steps)])) for j, n in enumerate(names)}
    ms_per_step = wall * 1e3 / args.steps

    # ---- algorithmic work of one step (see the kernel notes in the design doc) ----
    seg = np.diff(offsets.cpu().numpy())
    touched = int((seg > 0).sum())
    # bytes per element: MXFP8 codes + E8M0 scales; NVFP4 half-byte codes + E4M3 per 16
    eb = {"f32": 4, "bf16": 2, "mxfp8": 1 + 1 / 32, "nvfp4": 0.5 + 1 / 16}[wl.dtype]
    hb = eb
    ob = 4 if dt == pg.MOE_F32 else 2
    n_mats = touched + (1 if has_shared else 0)
    mat = I * d * eb
    bytes_gate_up = n_mats * 2 * mat + T * d * eb + rows * I * hb + T * k * 4
    bytes_down = n_mats * mat + rows * I * hb + rows * d * ob
    xb = 2 if wl.dtype == "nvfp4" else eb       # x as the layer takes it
    bytes_route = T * d * xb + d * E * 4 + T * k * 8 + (E * 4 if bias is not None else 0)
    if filt is not None:
        bytes_route += T * k * 4        # the replayed ids read besides the filtered ids written
    bytes_dispatch = T * k * 4 * 3 + (E + 1) * 4
    bytes_combine = rows * d * ob + T * d * ob + T * k * 8
    flops_gate_up = 2.0 * rows * d * 2 * I
    flops_down = 2.0 * rows * I * d
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9  # noqa: E731
    stages = {
        "route": {"ms": stage_ms["route"], "alg_bytes": bytes_route, "GB_s": gbs(bytes_route, stage_ms["route"])},
        "dispatch": {"ms": stage_ms["dispatch"], "alg_bytes": bytes_dispatch,
                     "GB_s": gbs(bytes_dispatch, stage_ms["dispatch"])},
        "ffn_gate_up": {"ms": stage_ms["ffn_gate_up"], "alg_bytes": bytes_gate_up,
                        "GB_s": gbs(bytes_gate_up, stage_ms["ffn_gate_up"]),
                        "TFLOP_s": flops_gate_up / (stage_ms["ffn_gate_up"] * 1e-3) / 1e12},
        "ffn_down": {"ms": stage_ms["ffn_down"], "alg_bytes": bytes_down,
                     "GB_s": gbs(bytes_down, stage_ms["ffn_down"]),
                     "TFLOP_s": flops_down / (stage_ms["ffn_down"] * 1e-3) / 1e12},
        "combine": {"ms": stage_ms["combine"], "alg_bytes": bytes_combine,
                    "GB_s": gbs(bytes_combine, stage_ms["combine"])},
    }
    if bwd:
        n_all = E + (1 if has_shared else 0)      # the weights half writes every expert's gradients
        bytes_cbwd = T * d * ob + T * k * d * ob * 2 + (T * d * ob if has_shared else 0) + T * k * 12
        bytes_data = (n_mats * 3 * mat + rows * 2 * I * 4 + rows * d * ob
                      + rows * 2 * I * 2 * 2 + rows * I * 2 + rows * d * 4)
        bytes_wts = n_all * 3 * I * d * 4 + rows * d * ob + rows * I * 2 + rows * 2 * I * 2 + rows * d * eb
        bytes_rbwd = rows * d * 4 + T * d * 4 + 2 * E * d * 4 + d * E * 4 + T * k * d * eb + T * k * 16
        flops_data = 2.0 * rows * d * I * 3
        stages["ffn_gate_up"]["alg_bytes"] += rows * 2 * I * 4   # the saved pre-activations
        stages["ffn_gate_up"]["GB_s"] = gbs(stages["ffn_gate_up"]["alg_bytes"], stage_ms["ffn_gate_up"])
        flops_wts = 2.0 * rows * d * I * 3
        parts = [("combine_backward", bytes_cbwd, None), ("route_backward", bytes_rbwd, None)]
        if mxb:
            # MXFP8 expert backward, one call: the requantised weights (fp8 + scales), the saved
            # pre-activations, d_out, x, the dx rows written and every expert's fp32 gradients
            bytes_mxb = (n_mats * 3 * mat + rows * 2 * I * 4 + rows * d * ob + T * d * eb + rows * d * 4
                         + n_all * 3 * I * d * 4)
            parts.append(("ffn_backward", bytes_mxb, flops_data + flops_wts))
        else:
            parts += [("ffn_backward_data", bytes_data, flops_data), ("ffn_backward_weights", bytes_wts, flops_wts)]
        for n, b, f in parts:
            stages[n] = {"ms": stage_ms[n], "alg_bytes": b, "GB_s": gbs(b, stage_ms[n])}
            if f is not None:
                stages[n]["TFLOP_s"] = f / (stage_ms[n] * 1e-3) / 1e12
    dom = max(("ffn_gate_up", "ffn_down"), key=lambda n: stage_ms[n])
    # the MXFP8 GEMMs run on the LDS-ring kernel where d and I are multiples of 512
    mx_ring = d % 512 == 0 and I % 512 == 0
    kname = {"f32": "grouped_ffn_f32_kernel", "bf16": "grouped_gemm_bf16_kernel",
             "mxfp8": "grouped_gemm_mx_ring_kernel" if mx_ring else "grouped_gemm_mx_kernel",
             "nvfp4": "grouped_gemm_fp4_kernel"}[wl.dtype]
    dom_kernel = {"ffn_gate_up": f"{kname}<0> (W1/W3 + SwiGLU)", "ffn_down": f"{kname}<1> (W2)"}[dom]
    gemm_tflops = (flops_gate_up + flops_down) / ((stage_ms["ffn_gate_up"] + stage_ms["ffn_down"]) * 1e-3) / 1e12
    mfma_peak = MXFP8_MFMA_PEAK_TFLOPS if wl.dtype == "mxfp8" else BF16_MFMA_PEAK_TFLOPS
    # Weight streaming bounds the grouped GEMMs when tokens per expert are few (the
    # bf16 workloads); the MXFP8 prefill chunk is bound by the block-scaled matrix cores.
    # NVFP4 operands are decoded to bf16 for the bf16 matrix cores: their peak is bf16's,
    # and at 0.56 byte per weight the matrix cores, not HBM, bound the GEMMs
    if wl.dtype in ("mxfp8", "nvfp4"):
        dom_flops = flops_gate_up if dom == "ffn_gate_up" else flops_down
        achieved = dom_flops / (stage_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": achieved / mfma_peak}
    else:
        achieved = stages[dom]["GB_s"]
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}

    if mxb:
        # the expert backward: MXFP8 GEMMs, bound by its HBM traffic (every expert's fp32
        # gradients dominate it)
        bdom = "ffn_backward"
        call = "moe_expert_ffn_backward_nvfp4" if wl.dtype == "nvfp4" else "moe_expert_ffn_backward_mxfp8"
        dom_kernel = (f"{call}: mx_bwd_gemm_kernel<0..2> + MX quantisers (dh, dx; "
                      "dW2, dW1 | dW3 of every expert)")
    if bwd and not mxb:
        # the step's largest stage is one of the two backward halves; both stream HBM
        bdom = max(("ffn_backward_data", "ffn_backward_weights"), key=lambda n: stage_ms[n])
        dom_kernel = {"ffn_backward_data": "bwd_gemm_kernel<0>/<1> + recompute (dx half: "
                                           "a, g; dh with SwiGLU backward; dx rows)",
                      "ffn_backward_weights": "bwd_gemm_kernel<2>, <3> (dW2; dW1 and dW3, fp32 "
                                              "gradients of every expert)"}[bdom]
    if bwd:
        achieved = stages[bdom]["GB_s"]
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
        dom = bdom
    result = {
        "metric": METRIC if not bwd else f"MoE-layer forward+backward tokens/s, 384-expert top-8 d=7168 {wl.dtype}",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "d": d, "E": E, "k": k, "inter": I,
                   "shared_experts": 1 if has_shared else 0, "routing": wl.routing,
                   "seed": wl.seed, "parallelism": "none (1 GPU)",
                   **({"replay_filter_log_tau": filt} if filt is not None else {})},
        "roofline": dict(roof, traffic=None, kernel=dom_kernel,
                         alg_bytes_per_launch=stages[dom]["alg_bytes"], launch_ms=stage_ms[dom]),
        "mfma": {"gemm_TFLOP_s": gemm_tflops, "peak_TFLOP_s": mfma_peak,
                 "frac": gemm_tflops / mfma_peak,
                 "flops_per_step": flops_gate_up + flops_down},
        "stages": stages,
        "experts_touched": touched,
        "input_draw_s": t_draw,
    }

    result["roofline"]["traffic"] = measured_traffic(wl.name) if dom == "ffn_gate_up" else None
    counters = measured_mfma(wl.name)
    if counters is not None:
        result["mfma"]["counters"] = counters
    if bwd:
        result["config"]["pass"] = "forward+backward"
    if wl.dtype != "bf16":
        result["vs_metric_config"] = "this workload is not the metric's configuration (bf16 T=4096)"
    if wl.dtype == "nvfp4":
        result["config"]["experts"] = "NVFP4 (E2M1, E4M3 per 16, fp32 per row); x, y bf16"
    if bwd:   # the oracle's backward keeps every touched expert's fp64 gradients: few tokens
        args.cpu_sample = min(args.cpu_sample, 4)
    if args.cpu_sample > 0:
        result["cpu_baseline"] = cpu_baseline(inp, wl, ids, args.cpu_sample, filt,
                                              dy if bwd else None)
    print(json.dumps(result))


def _sources_sha(files):
    """SHA-256 of the kernel's source files (the .hip file and the headers it includes),
    concatenated in the listed order."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "parity_gate_gemm_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 FETCH_SIZE + WRITE_SIZE
    summary (each scaled by the plain-copy calibration), or None when no summary exists
    for this workload or the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"gemm1_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if "kernel_sources" not in rec or _sources_sha(rec["kernel_sources"]) != rec["sources_sha256"]:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def measured_mfma(workload):
    """Matrix-core counters of the grouped GEMMs from the committed rocprofv3 summary
    (SQ_VALU_MFMA_BUSY_CYCLES over the SIMD cycles, the implied clock, the counted
    matrix operations), or None when there is none or the kernel source changed."""
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if "kernel_sources" not in rec or _sources_sha(rec["kernel_sources"]) != rec["sources_sha256"]:
        return None
    return {k: {"mfma_busy": round(v["mfma_busy"], 4), "clock_ghz": round(v["clock_ghz"], 3),
                "mfma_ops": v["ops"]} for k, v in rec["kernels"].items() if "grouped_gemm" in k}


class _ExpertCache:
    """experts[e] -> host arrays of the stored values.  The device-to-host copies are
    made before the oracle is timed; the widening to fp32 is part of the timed work."""

    def __init__(self, inp):
        self.inp = inp
        self.cache = {}

    def fetch(self, e):
        if e not in self.cache:
            self.cache[e] = tuple(tuple(None if self.inp.get(n + sfx) is None else self.inp[n + sfx][e].cpu()
                                        for sfx in ("", "_scale", "_rscale"))
                                  for n in ("w1", "w3", "w2"))
        return self.cache[e]

    def __getitem__(self, e):
        return tuple(_stored_values(*m) for m in self.fetch(e))


def _stored_values(t, scale=None, rscale=None):
    """Host values of a stored tensor (MXFP8 codes decoded by the oracle's decoder); an
    NVFP4 matrix stays the (codes, block scales, row scales) triple the oracle takes."""
    import numpy as np
    import oracle
    if rscale is not None:
        p = t.numpy()
        codes = np.stack([p & 15, p >> 4], axis=-1).reshape(p.shape[0], -1)
        return codes, scale.numpy(), rscale.numpy()
    if scale is None:
        return t.float().numpy()
    return oracle.mx_dequant(t.numpy(), scale.numpy())


def cpu_baseline(inp, wl, ids, n_tok, log_tau=None, dy=None):
    """The CPU oracle (as it is) on the first n_tok tokens of the same batch; with
    log_tau, the filtered replay routing followed by the layer on the filtered ids."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    rows = np.arange(min(n_tok, wl.T))
    xs = inp["x_scale"]
    x = _stored_values(inp["x"][rows].cpu(), None if xs is None else xs[rows].cpu())
    wg = inp["w_gate"].cpu().numpy()
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    experts = _ExpertCache(inp)
    for e in np.unique(ids[rows].cpu().numpy()):
        experts.fetch(int(e))                       # host copies: not part of the timed work
    sh = inp["shared"]
    shared = None if sh is None else tuple(
        _stored_values(*(None if sh.get(n + sfx) is None else sh[n + sfx].cpu() for sfx in ("", "_scale", "_rscale")))
        for n in ("w1", "w3", "w2"))
    kw = {}
    if wl.routing == "replay":
        kw = {"ids_in": inp["ids_in"][rows].cpu().numpy(), "weights_in": inp["weights_in"][rows].cpu().numpy()}
    t0 = time.perf_counter()
    if log_tau is not None:
        fid, fw, _, _ = oracle.route_replay_filtered(x, wg, bias, kw["ids_in"], log_tau)
        kw = {"ids_in": fid, "weights_in": fw}
    if wl.dtype == "nvfp4" and dy is None:
        oracle.layer_nvfp4(x, wg, bias, experts, shared, wl.k, **kw)
    elif dy is None:
        oracle.layer(x, wg, bias, experts, shared, wl.k, **kw)
    elif wl.dtype in ("mxfp8", "nvfp4"):
        oracle.layer_backward_mxfp8(x, wg, bias, experts, shared, wl.k, dy[rows].float().cpu().numpy(),
                                    forward=wl.dtype, **kw)
    else:
        oracle.layer_backward(x, wg, bias, experts, shared, wl.k, dy[rows].float().cpu().numpy(),
                              dense=False, **kw)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {len(rows)} tokens of the {wl.name} batch (exact fsum gate logits over "
                      f"{wl.E} experts{', plausibility filter' if log_tau is not None else ''}, fp64 "
                      f"SwiGLU for each chosen expert{', then its fp64 backward' if dy is not None else ''}), "
                      f"{dt:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
