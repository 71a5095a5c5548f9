"""Python binding of libmoe (the C ABI in include/moe.h) over torch tensors.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe.so``.  Tensors must already live on the GPU; the binding passes their
device pointers and the current HIP stream.  There is no fallback: if the library
is not built, importing the call table raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MOE_F32", "MOE_BF16", "MOE_MXFP8", "MOE_NVFP4", "MoeError", "moe_nvfp4_quantize",
    "moe_nvfp4_pack_weights", "nvfp4_pack_inputs", "lib", "Workspace",
    "moe_workspace_size", "moe_workspace_init", "moe_route", "moe_route_replay",
    "moe_route_replay_filtered",
    "moe_dispatch", "moe_dispatch_noalloc", "moe_expert_ffn", "moe_expert_ffn_gate_up", "moe_expert_ffn_down", "moe_combine", "moe_check", "moe_status_string",
    "layer_forward", "moe_backward_workspace_size", "moe_combine_backward", "moe_expert_ffn_backward",
    "moe_route_backward", "layer_backward", "moe_expert_ffn_backward_data",
    "moe_expert_ffn_backward_weights", "moe_expert_ffn_gate_up_save", "moe_mxfp8_transpose_weights",
    "moe_expert_ffn_backward_mxfp8", "moe_nvfp4_transpose_weights", "moe_expert_ffn_backward_nvfp4",
]

MOE_F32, MOE_BF16, MOE_MXFP8, MOE_NVFP4 = 0, 1, 2, 3
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_string(status)}")


class _Bank(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w1_scale", ctypes.c_void_p), ("w3_scale", ctypes.c_void_p),
                ("w2_scale", ctypes.c_void_p), ("w1_rscale", ctypes.c_void_p),
                ("w3_rscale", ctypes.c_void_p), ("w2_rscale", ctypes.c_void_p)]


class _GradBank(ctypes.Structure):
    _fields_ = [("dw1", ctypes.c_void_p), ("dw3", ctypes.c_void_p), ("dw2", ctypes.c_void_p)]


class _TBank(ctypes.Structure):
    _fields_ = [("w2t", ctypes.c_void_p), ("w2t_scale", ctypes.c_void_p), ("w13t", ctypes.c_void_p),
                ("w13t_scale", ctypes.c_void_p)]


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmoe.so not found at {LIB_PATH}; build it with "
                              "`python -m parity_gate_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, SZ, PSZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)
        sig = {
            "moe_workspace_size": [I, I, I, I, I, I, PSZ],
            "moe_workspace_init": [P, SZ, P],
            "moe_route": [P, P, I, I, I, P, P, I, I, P, P, P, SZ, P],
            "moe_route_replay": [P, P, I, I, I, P, P, I, I, P, P, P, P, SZ, P],
            "moe_backward_workspace_size": [I, I, I, I, I, I, PSZ],
            "moe_nvfp4_quantize": [P, I, I, P, P, P, P],
            "moe_nvfp4_pack_weights": [P, P, I, I, I, P, P, P],
            "moe_combine_backward": [P, I, P, P, P, I, I, I, I, P, P, P],
            "moe_expert_ffn_backward": [P, P, I, I, I, I, I, I, ctypes.POINTER(_Bank),
                                        ctypes.POINTER(_Bank), P, P, P, P, P, ctypes.POINTER(_GradBank),
                                        ctypes.POINTER(_GradBank), P, SZ, P],
            "moe_expert_ffn_gate_up_save": [P, P, I, I, I, I, I, I, ctypes.POINTER(_Bank),
                                            ctypes.POINTER(_Bank), P, P, P, P, SZ, P],
            "moe_expert_ffn_backward_data": [P, P, I, I, I, I, I, I, ctypes.POINTER(_Bank),
                                             ctypes.POINTER(_Bank), P, P, P, P, P, P, SZ, P],
            "moe_expert_ffn_backward_weights": [P, I, I, I, I, I, I, ctypes.POINTER(_Bank),
                                                ctypes.POINTER(_Bank), P, P, ctypes.POINTER(_GradBank),
                                                ctypes.POINTER(_GradBank), P, SZ, P],
            "moe_route_backward": [P, P, I, I, I, P, I, I, P, P, P, P, P, P, P, I, P, P, P, P, SZ, P],
            "moe_route_replay_filtered": [P, P, I, I, I, P, P, I, I, P, ctypes.c_double, P, P, P, SZ,
                                          P],
            "moe_dispatch": [P, I, I, I, P, P, P, P, SZ, P],
            "moe_dispatch_noalloc": [P, I, I, I, P, P, P, P, P],
            "moe_mxfp8_transpose_weights": [ctypes.POINTER(_Bank), I, I, I, ctypes.POINTER(_TBank), P],
            "moe_nvfp4_transpose_weights": [ctypes.POINTER(_Bank), I, I, I, ctypes.POINTER(_TBank), P],
            "moe_expert_ffn_backward_nvfp4": [P, I, I, I, I, I, ctypes.POINTER(_Bank), ctypes.POINTER(_Bank),
                                              ctypes.POINTER(_TBank), ctypes.POINTER(_TBank), P, P, P, P, P,
                                              ctypes.POINTER(_GradBank), ctypes.POINTER(_GradBank), P, SZ, P],
            "moe_expert_ffn_backward_mxfp8": [P, P, I, I, I, I, I, ctypes.POINTER(_Bank), ctypes.POINTER(_Bank),
                                              ctypes.POINTER(_TBank), ctypes.POINTER(_TBank), P, P, P, P, P,
                                              ctypes.POINTER(_GradBank), ctypes.POINTER(_GradBank), P, SZ, P],
            "moe_expert_ffn": [P, P, I, I, I, I, I, I, ctypes.POINTER(_Bank), ctypes.POINTER(_Bank),
                               P, P, P, P, SZ, P],
            "moe_expert_ffn_gate_up": [P, P, I, I, I, I, I, I, ctypes.POINTER(_Bank),
                                       ctypes.POINTER(_Bank), P, P, P, SZ, P],
            "moe_expert_ffn_down": [I, I, I, I, I, I, ctypes.POINTER(_Bank), ctypes.POINTER(_Bank),
                                    P, P, SZ, P],
            "moe_combine": [P, I, P, P, I, I, I, I, P, P],
            "moe_check": [P, SZ, P],
            "moe_status_string": [I],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "moe_status_string" else ctypes.c_int
        _lib = L
    return _lib


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _ok(status: int, where: str):
    if status != 0:
        raise MoeError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_of(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return MOE_F32
    if x.dtype == torch.bfloat16:
        return MOE_BF16
    if x.dtype == torch.uint8:
        return MOE_MXFP8
    raise TypeError(f"unsupported activation dtype {x.dtype}")


def _check_dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libmoe takes device tensors only")
            if not t.is_contiguous():
                raise ValueError("libmoe takes contiguous (row-major) tensors only")


def moe_workspace_size(T: int, d: int, E: int, k: int, inter: int, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    _ok(lib().moe_workspace_size(T, d, E, k, inter, dtype, ctypes.byref(n)), "moe_workspace_size")
    return n.value


def moe_workspace_init(ws: torch.Tensor):
    _ok(lib().moe_workspace_init(_ptr(ws), ws.numel(), _stream(ws.device)), "moe_workspace_init")


class Workspace:
    """A device workspace sized for one layer shape, with its header initialised."""

    def __init__(self, T, d, E, k, inter, dtype, device="cuda"):
        self.nbytes = moe_workspace_size(T, d, E, k, inter, dtype)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        moe_workspace_init(self.buf)

    @property
    def ptr(self):
        return _ptr(self.buf)


def moe_route(x, w_gate, bias, k, ws: Workspace, x_scale=None, ids=None, weights=None):
    _check_dev(x, w_gate, bias, x_scale)
    T, d = x.shape
    E = w_gate.shape[1]
    ids = torch.empty(T, k, dtype=torch.int32, device=x.device) if ids is None else ids
    weights = torch.empty(T, k, dtype=torch.float32, device=x.device) if weights is None else weights
    _ok(lib().moe_route(_ptr(x), _ptr(x_scale), _dtype_of(x), T, d, _ptr(w_gate), _ptr(bias), E, k,
                        _ptr(ids), _ptr(weights), ws.ptr, ws.nbytes, _stream(x.device)), "moe_route")
    return ids, weights


def moe_route_replay(x, w_gate, bias, ids_in, ws: Workspace, weights_in=None, x_scale=None,
                     weights_out=None):
    _check_dev(x, w_gate, bias, x_scale, ids_in, weights_in)
    T, d = x.shape
    E = w_gate.shape[1]
    k = ids_in.shape[1]
    wo = torch.empty(T, k, dtype=torch.float32, device=x.device) if weights_out is None else weights_out
    _ok(lib().moe_route_replay(_ptr(x), _ptr(x_scale), _dtype_of(x), T, d, _ptr(w_gate), _ptr(bias),
                               E, k, _ptr(ids_in), _ptr(weights_in), _ptr(wo), ws.ptr, ws.nbytes,
                               _stream(x.device)), "moe_route_replay")
    return wo


def moe_route_replay_filtered(x, w_gate, bias, ids_in, log_tau, ws: Workspace, x_scale=None,
                              ids_out=None, weights_out=None):
    _check_dev(x, w_gate, bias, x_scale, ids_in)
    T, d = x.shape
    E = w_gate.shape[1]
    k = ids_in.shape[1]
    io = torch.empty(T, k, dtype=torch.int32, device=x.device) if ids_out is None else ids_out
    wo = torch.empty(T, k, dtype=torch.float32, device=x.device) if weights_out is None else weights_out
    _ok(lib().moe_route_replay_filtered(_ptr(x), _ptr(x_scale), _dtype_of(x), T, d, _ptr(w_gate),
                                        _ptr(bias), E, k, _ptr(ids_in), float(log_tau), _ptr(io),
                                        _ptr(wo), ws.ptr, ws.nbytes, _stream(x.device)),
        "moe_route_replay_filtered")
    return io, wo


def moe_dispatch(ids, E, ws: Workspace, offsets=None, perm=None, row_of=None):
    _check_dev(ids)
    T, k = ids.shape
    dev = ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    perm = torch.empty(T * k, dtype=torch.int32, device=dev) if perm is None else perm
    row_of = torch.empty(T * k, dtype=torch.int32, device=dev) if row_of is None else row_of
    _ok(lib().moe_dispatch(_ptr(ids), T, E, k, _ptr(offsets), _ptr(perm), _ptr(row_of), ws.ptr,
                           ws.nbytes, _stream(dev)), "moe_dispatch")
    return offsets, perm, row_of


def moe_dispatch_noalloc(ids, E, offsets=None, perm=None, row_of=None, status=None):
    """moe_dispatch on the library's static scratch (no workspace); ``status`` is an
    optional int32 device tensor of one element that receives the device status."""
    _check_dev(ids)
    T, k = ids.shape
    dev = ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    perm = torch.empty(T * k, dtype=torch.int32, device=dev) if perm is None else perm
    row_of = torch.empty(T * k, dtype=torch.int32, device=dev) if row_of is None else row_of
    _ok(lib().moe_dispatch_noalloc(_ptr(ids), T, E, k, _ptr(offsets), _ptr(perm), _ptr(row_of),
                                   _ptr(status), _stream(dev)), "moe_dispatch_noalloc")
    return offsets, perm, row_of


_BANK_OPT = ("w1_scale", "w3_scale", "w2_scale", "w1_rscale", "w3_rscale", "w2_rscale")


def _bank(b):
    if b is None:
        return None
    _check_dev(b["w1"], b["w3"], b["w2"], *(b.get(n) for n in _BANK_OPT))
    return _Bank(b["w1"].data_ptr(), b["w3"].data_ptr(), b["w2"].data_ptr(),
                 *(b[n].data_ptr() if b.get(n) is not None else None for n in _BANK_OPT))


def _ffn_dtype(x, routed):
    """The expert FFN's dtype: NVFP4 when the weights carry row scales (x is bf16)."""
    return MOE_NVFP4 if routed.get("w1_rscale") is not None else _dtype_of(x)


def moe_expert_ffn(x, routed: dict, shared, offsets, perm, k, ws: Workspace, x_scale=None, out=None):
    """routed/shared: dicts with w1, w3, w2 (and *_scale for MXFP8); shared may be None."""
    _check_dev(x, x_scale, offsets, perm)
    T, d = x.shape
    E = routed["w1"].shape[0]
    inter = routed["w1"].shape[1]
    dt = _ffn_dtype(x, routed)
    rows = T * k + (T if shared is not None else 0)
    if out is None:
        out = torch.empty(rows, d, dtype=torch.float32 if dt == MOE_F32 else torch.bfloat16,
                          device=x.device)
    rb, sb = _bank(routed), _bank(shared)
    _ok(lib().moe_expert_ffn(_ptr(x), _ptr(x_scale), dt, T, d, E, k, inter, ctypes.byref(rb),
                             ctypes.byref(sb) if sb is not None else None, _ptr(offsets), _ptr(perm),
                             _ptr(out), ws.ptr, ws.nbytes, _stream(x.device)), "moe_expert_ffn")
    return out


def moe_expert_ffn_gate_up(x, routed: dict, shared, offsets, perm, k, ws: Workspace, x_scale=None):
    """GEMM1 half of moe_expert_ffn (h stays in the workspace)."""
    _check_dev(x, x_scale, offsets, perm)
    T, d = x.shape
    E, inter = routed["w1"].shape[0], routed["w1"].shape[1]
    rb, sb = _bank(routed), _bank(shared)
    _ok(lib().moe_expert_ffn_gate_up(_ptr(x), _ptr(x_scale), _ffn_dtype(x, routed), T, d, E, k, inter,
                                     ctypes.byref(rb), ctypes.byref(sb) if sb is not None else None,
                                     _ptr(offsets), _ptr(perm), ws.ptr, ws.nbytes, _stream(x.device)),
        "moe_expert_ffn_gate_up")


def moe_expert_ffn_down(dtype, T, d, routed: dict, shared, k, ws: Workspace, out=None):
    """GEMM2 half of moe_expert_ffn, after moe_expert_ffn_gate_up on the same workspace."""
    E, inter = routed["w1"].shape[0], routed["w1"].shape[1]
    if routed.get("w1_rscale") is not None:
        dtype = MOE_NVFP4
    rows = T * k + (T if shared is not None else 0)
    dev = routed["w1"].device
    if out is None:
        out = torch.empty(rows, d, dtype=torch.float32 if dtype == MOE_F32 else torch.bfloat16, device=dev)
    _check_dev(out)
    rb, sb = _bank(routed), _bank(shared)
    _ok(lib().moe_expert_ffn_down(dtype, T, d, E, k, inter, ctypes.byref(rb),
                                  ctypes.byref(sb) if sb is not None else None, _ptr(out), ws.ptr,
                                  ws.nbytes, _stream(dev)), "moe_expert_ffn_down")
    return out


def moe_combine(out, row_of, weights, T, has_shared, dtype, y=None):
    _check_dev(out, row_of, weights)
    d = out.shape[1]
    k = weights.shape[1] if weights.dim() == 2 else 1
    if y is None:
        y = torch.empty(T, d, dtype=torch.float32 if dtype == MOE_F32 else torch.bfloat16,
                        device=out.device)
    _ok(lib().moe_combine(_ptr(out), dtype, _ptr(row_of), _ptr(weights), T, d, k,
                          1 if has_shared else 0, _ptr(y), _stream(out.device)), "moe_combine")
    return y


def moe_check(ws: Workspace) -> int:
    """Synchronises, reads and clears the device error flag; returns the status code."""
    return lib().moe_check(ws.ptr, ws.nbytes, _stream(ws.buf.device))


def layer_forward(inp: dict, k: int, ws: Workspace | None = None, replay: bool = False,
                  check: bool = True, save_pre: bool = False):
    """One MoE layer forward through the five C calls.

    ``inp`` holds device tensors: x, x_scale, w_gate, bias, w1, w3, w2 (+ *_scale),
    shared (dict or None) and, for replay, ids_in / weights_in.  With ``save_pre`` the
    expert FFN runs as its two halves, the first keeping the fp32 pre-activations for
    the backward (returned as "pre").
    """
    x = inp["x"]
    T, d = x.shape
    E = inp["w_gate"].shape[1]
    inter = inp["w1"].shape[1]
    dt = _dtype_of(x)
    if ws is None:
        fdt = MOE_NVFP4 if inp.get("w1_rscale") is not None else dt
        ws = Workspace(T, d, E, k, inter, fdt, device=x.device)
    if replay:
        ids = inp["ids_in"]
        weights = moe_route_replay(x, inp["w_gate"], inp.get("bias"), ids, ws,
                                   weights_in=inp.get("weights_in"), x_scale=inp.get("x_scale"))
    else:
        ids, weights = moe_route(x, inp["w_gate"], inp.get("bias"), k, ws, x_scale=inp.get("x_scale"))
    offsets, perm, row_of = moe_dispatch(ids, E, ws)
    routed = {n: inp.get(n) for n in ("w1", "w3", "w2") + _BANK_OPT}
    pre = None
    if save_pre:
        pre = moe_expert_ffn_gate_up_save(x, routed, inp.get("shared"), offsets, perm, k, ws,
                                          x_scale=inp.get("x_scale"))
        out = moe_expert_ffn_down(dt, T, d, routed, inp.get("shared"), k, ws)
    else:
        out = moe_expert_ffn(x, routed, inp.get("shared"), offsets, perm, k, ws, x_scale=inp.get("x_scale"))
    y = moe_combine(out, row_of, weights, T, inp.get("shared") is not None, dt)
    if check:
        st = moe_check(ws)
        if st != 0:
            raise MoeError(st, "layer_forward")
    return {"y": y, "ids": ids, "weights": weights, "offsets": offsets, "perm": perm,
            "row_of": row_of, "out": out, "pre": pre}


# ---------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------
def moe_backward_workspace_size(T, d, E, k, inter, dtype) -> int:
    n = ctypes.c_size_t()
    _ok(lib().moe_backward_workspace_size(T, d, E, k, inter, dtype, ctypes.byref(n)),
        "moe_backward_workspace_size")
    return n.value


class BackwardWorkspace(Workspace):
    """A workspace sized for the forward and the backward calls of one layer shape."""

    def __init__(self, T, d, E, k, inter, dtype, device="cuda"):
        self.nbytes = moe_backward_workspace_size(T, d, E, k, inter, dtype)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        moe_workspace_init(self.buf)


def moe_combine_backward(dy, out, row_of, weights, T, has_shared, dtype, d_out=None, d_weights=None):
    _check_dev(dy, out, row_of, weights)
    d = out.shape[1]
    k = weights.shape[1]
    d_out = torch.empty_like(out) if d_out is None else d_out
    d_weights = torch.empty(T, k, dtype=torch.float32, device=out.device) if d_weights is None else d_weights
    _ok(lib().moe_combine_backward(_ptr(dy), dtype, _ptr(out), _ptr(row_of), _ptr(weights), T, d, k,
                                   1 if has_shared else 0, _ptr(d_out), _ptr(d_weights),
                                   _stream(out.device)), "moe_combine_backward")
    return d_out, d_weights


def _grads(b):
    return None if b is None else _GradBank(b["w1"].data_ptr(), b["w3"].data_ptr(), b["w2"].data_ptr())


def _grad_like(bank):
    return {n: torch.empty(bank[n].shape, dtype=torch.float32, device=bank[n].device)
            for n in ("w1", "w3", "w2")}


def moe_expert_ffn_gate_up_save(x, routed: dict, shared, offsets, perm, k, ws: Workspace, pre=None,
                                x_scale=None):
    """GEMM1 half that also returns the fp32 pre-activations [rows][2I] for the backward."""
    _check_dev(x, offsets, perm, x_scale)
    T, d = x.shape
    E, inter = routed["w1"].shape[0], routed["w1"].shape[1]
    rows = T * k + (T if shared is not None else 0)
    pre = torch.empty(rows, 2 * inter, dtype=torch.float32, device=x.device) if pre is None else pre
    rb, sb = _bank(routed), _bank(shared)
    _ok(lib().moe_expert_ffn_gate_up_save(_ptr(x), _ptr(x_scale), _ffn_dtype(x, routed), T, d, E, k, inter,
                                          ctypes.byref(rb),
                                          ctypes.byref(sb) if sb is not None else None, _ptr(offsets),
                                          _ptr(perm), _ptr(pre), ws.ptr, ws.nbytes, _stream(x.device)),
        "moe_expert_ffn_gate_up_save")
    return pre


def moe_expert_ffn_backward(x, routed: dict, shared, offsets, perm, k, d_out, ws: Workspace,
                            x_scale=None, dx_rows=None, grads=None, shared_grads=None, pre=None):
    """Returns (dx_rows [rows][d] fp32, grads {w1, w3, w2} fp32, shared grads or None)."""
    _check_dev(x, x_scale, offsets, perm, d_out)
    T, d = x.shape
    E, inter = routed["w1"].shape[0], routed["w1"].shape[1]
    rows = T * k + (T if shared is not None else 0)
    dx_rows = torch.empty(rows, d, dtype=torch.float32, device=x.device) if dx_rows is None else dx_rows
    grads = _grad_like(routed) if grads is None else grads
    if shared is not None and shared_grads is None:
        shared_grads = _grad_like(shared)
    rb, sb = _bank(routed), _bank(shared)
    rg, sg = _grads(grads), _grads(shared_grads)
    _ok(lib().moe_expert_ffn_backward(_ptr(x), _ptr(x_scale), _dtype_of(x), T, d, E, k, inter,
                                      ctypes.byref(rb), ctypes.byref(sb) if sb is not None else None,
                                      _ptr(offsets), _ptr(perm), _ptr(pre), _ptr(d_out), _ptr(dx_rows),
                                      ctypes.byref(rg), ctypes.byref(sg) if sg is not None else None,
                                      ws.ptr, ws.nbytes, _stream(x.device)), "moe_expert_ffn_backward")
    return dx_rows, grads, shared_grads


def moe_expert_ffn_backward_data(x, routed: dict, shared, offsets, perm, k, d_out, ws: Workspace,
                                 x_scale=None, dx_rows=None, pre=None):
    _check_dev(x, x_scale, offsets, perm, d_out)
    T, d = x.shape
    E, inter = routed["w1"].shape[0], routed["w1"].shape[1]
    rows = T * k + (T if shared is not None else 0)
    dx_rows = torch.empty(rows, d, dtype=torch.float32, device=x.device) if dx_rows is None else dx_rows
    rb, sb = _bank(routed), _bank(shared)
    _ok(lib().moe_expert_ffn_backward_data(_ptr(x), _ptr(x_scale), _dtype_of(x), T, d, E, k, inter,
                                           ctypes.byref(rb), ctypes.byref(sb) if sb is not None else None,
                                           _ptr(offsets), _ptr(perm), _ptr(pre), _ptr(d_out), _ptr(dx_rows),
                                           ws.ptr,
                                           ws.nbytes, _stream(x.device)), "moe_expert_ffn_backward_data")
    return dx_rows


def moe_expert_ffn_backward_weights(x, routed: dict, shared, perm, k, d_out, ws: Workspace, grads=None,
                                    shared_grads=None):
    _check_dev(x, perm, d_out)
    T, d = x.shape
    E, inter = routed["w1"].shape[0], routed["w1"].shape[1]
    grads = _grad_like(routed) if grads is None else grads
    if shared is not None and shared_grads is None:
        shared_grads = _grad_like(shared)
    rb, sb = _bank(routed), _bank(shared)
    rg, sg = _grads(grads), _grads(shared_grads)
    _ok(lib().moe_expert_ffn_backward_weights(_ptr(x), _dtype_of(x), T, d, E, k, inter, ctypes.byref(rb),
                                              ctypes.byref(sb) if sb is not None else None, _ptr(perm),
                                              _ptr(d_out), ctypes.byref(rg),
                                              ctypes.byref(sg) if sg is not None else None, ws.ptr,
                                              ws.nbytes, _stream(x.device)), "moe_expert_ffn_backward_weights")
    return grads, shared_grads


def moe_route_backward(x, w_gate, ids, weights, d_weights, offsets, perm, row_of, dx_rows, has_shared,
                       ws: Workspace, gate_grad=True, bias_grad=True, x_scale=None, dx=None):
    """Returns (dx [T][d] fp32, d_w_gate [d][E] or None, d_bias [E] or None)."""
    _check_dev(x, x_scale, w_gate, ids, weights, d_weights, offsets, perm, row_of, dx_rows)
    T, d = x.shape
    E = w_gate.shape[1]
    k = ids.shape[1]
    dev = x.device
    dx = torch.empty(T, d, dtype=torch.float32, device=dev) if dx is None else dx
    dwg = torch.empty(d, E, dtype=torch.float32, device=dev) if gate_grad else None
    db = torch.empty(E, dtype=torch.float32, device=dev) if gate_grad and bias_grad else None
    _ok(lib().moe_route_backward(_ptr(x), _ptr(x_scale), _dtype_of(x), T, d, _ptr(w_gate), E, k,
                                 _ptr(ids), _ptr(weights), _ptr(d_weights), _ptr(offsets), _ptr(perm),
                                 _ptr(row_of), _ptr(dx_rows), 1 if has_shared else 0, _ptr(dx),
                                 _ptr(dwg), _ptr(db), ws.ptr, ws.nbytes, _stream(dev)),
        "moe_route_backward")
    return dx, dwg, db


def layer_backward(inp: dict, k: int, fwd: dict, dy, ws: Workspace, replay: bool = False,
                   check: bool = True, pre=None):
    """Gradients of one layer through the three backward C calls, given the forward's
    routing/dispatch results and expert outputs (``layer_forward``'s dict) and dL/dy.
    The gate gets a gradient unless the routing weights were the caller's."""
    x = inp["x"]
    T = x.shape[0]
    dt = _dtype_of(x)
    has_shared = inp.get("shared") is not None
    d_out, d_weights = moe_combine_backward(dy, fwd["out"], fwd["row_of"], fwd["weights"], T, has_shared, dt)
    routed = {n: inp.get(n) for n in ("w1", "w3", "w2") + _BANK_OPT}
    if inp.get("w1_rscale") is not None:   # NVFP4 forward, MXFP8 backward
        rt = inp.get("routed_t") or moe_mxfp8_transpose_weights(routed)
        st = inp.get("shared_t") if inp.get("shared") is None or inp.get("shared_t") is not None else \
            moe_mxfp8_transpose_weights(inp["shared"])
        dx_rows, grads, sgrads = moe_expert_ffn_backward_nvfp4(x, routed, inp.get("shared"), rt, st, fwd["offsets"],
                                                               fwd["perm"], k, d_out, ws, pre)
    elif dt == MOE_MXFP8:   # the requantised weights: from the caller, else made here
        rt = inp.get("routed_t") or moe_mxfp8_transpose_weights(routed)
        st = inp.get("shared_t") if inp.get("shared") is None or inp.get("shared_t") is not None else \
            moe_mxfp8_transpose_weights(inp["shared"])
        dx_rows, grads, sgrads = moe_expert_ffn_backward_mxfp8(x, inp["x_scale"], routed, inp.get("shared"), rt,
                                                               st, fwd["offsets"], fwd["perm"], k, d_out, ws,
                                                               pre=pre)
    else:
        dx_rows, grads, sgrads = moe_expert_ffn_backward(x, routed, inp.get("shared"), fwd["offsets"],
                                                         fwd["perm"], k, d_out, ws, x_scale=inp.get("x_scale"),
                                                         pre=pre)
    gate_grad = not (replay and inp.get("weights_in") is not None)
    dx, dwg, db = moe_route_backward(x, inp["w_gate"], fwd["ids"], fwd["weights"], d_weights,
                                     fwd["offsets"], fwd["perm"], fwd["row_of"], dx_rows, has_shared, ws,
                                     gate_grad=gate_grad, bias_grad=inp.get("bias") is not None,
                                     x_scale=inp.get("x_scale"))
    if check:
        st = moe_check(ws)
        if st != 0:
            raise MoeError(st, "layer_backward")
    return {"dx": dx, "d_weights": d_weights, "d_w_gate": dwg, "d_bias": db, "grads": grads,
            "shared_grads": sgrads, "dx_rows": dx_rows, "d_out": d_out}


def moe_mxfp8_transpose_weights(bank: dict) -> dict:
    """The requantised weights of an MXFP8 bank (w1, w3 [n][I][d], w2 [n][d][I] with their
    scales; a shared bank may drop the leading n), or of a K-blocked NVFP4 bank (with row
    scales), for the MXFP8 backward: w2t [n][I][d], w13t [n][d][2I] and their scales."""
    _check_dev(*(bank.get(n) for n in ("w1", "w3", "w2") + _BANK_OPT))
    nv = bank.get("w1_rscale") is not None
    one = bank["w1"].dim() == 2
    w1 = bank["w1"].unsqueeze(0) if one else bank["w1"]
    n, inter, d = w1.shape
    d = d * 2 if nv else d          # NVFP4: two codes per byte
    dev = w1.device
    out = {"w2t": torch.empty(n, inter, d, dtype=torch.uint8, device=dev),
           "w2t_scale": torch.empty(n, inter, d // 32, dtype=torch.uint8, device=dev),
           "w13t": torch.empty(n, d, 2 * inter, dtype=torch.uint8, device=dev),
           "w13t_scale": torch.empty(n, d, 2 * inter // 32, dtype=torch.uint8, device=dev)}
    tb = _TBank(*(out[k].data_ptr() for k in ("w2t", "w2t_scale", "w13t", "w13t_scale")))
    fn = lib().moe_nvfp4_transpose_weights if nv else lib().moe_mxfp8_transpose_weights
    _ok(fn(ctypes.byref(_bank(bank)), n, d, inter, ctypes.byref(tb), _stream(dev)), "moe_*_transpose_weights")
    return {k: (v[0] if one else v) for k, v in out.items()}


def _tbank(t):
    if t is None:
        return None
    _check_dev(*t.values())
    return _TBank(*(t[k].data_ptr() for k in ("w2t", "w2t_scale", "w13t", "w13t_scale")))


def moe_expert_ffn_backward_mxfp8(x, x_scale, routed: dict, shared, routed_t: dict, shared_t, offsets, perm,
                                  k, d_out, ws: Workspace, pre=None, dx_rows=None, grads=None,
                                  shared_grads=None):
    """Returns (dx_rows [rows][d] fp32, grads {w1, w3, w2} fp32, shared grads or None)."""
    _check_dev(x, x_scale, offsets, perm, d_out, pre)
    T, d = x.shape
    E, inter = routed["w1"].shape[0], routed["w1"].shape[1]
    rows = T * k + (T if shared is not None else 0)
    dx_rows = torch.empty(rows, d, dtype=torch.float32, device=x.device) if dx_rows is None else dx_rows
    grads = _grad_like(routed) if grads is None else grads
    if shared is not None and shared_grads is None:
        shared_grads = _grad_like(shared)
    rb, sb = _bank(routed), _bank(shared)
    rt, st = _tbank(routed_t), _tbank(shared_t)
    rg, sg = _grads(grads), _grads(shared_grads)
    ref = lambda v: ctypes.byref(v) if v is not None else None  # noqa: E731
    _ok(lib().moe_expert_ffn_backward_mxfp8(_ptr(x), _ptr(x_scale), T, d, E, k, inter, ref(rb), ref(sb), ref(rt),
                                            ref(st), _ptr(offsets), _ptr(perm), _ptr(pre), _ptr(d_out),
                                            _ptr(dx_rows), ref(rg), ref(sg), ws.ptr, ws.nbytes, _stream(x.device)),
        "moe_expert_ffn_backward_mxfp8")
    return dx_rows, grads, shared_grads


def moe_expert_ffn_backward_nvfp4(x, routed: dict, shared, routed_t: dict, shared_t, offsets, perm, k, d_out,
                                  ws: Workspace, pre, dx_rows=None, grads=None, shared_grads=None):
    """The MXFP8 backward of an NVFP4 layer (bf16 x, K-blocked NVFP4 banks, saved pre).
    Returns (dx_rows, grads, shared grads or None)."""
    _check_dev(x, offsets, perm, d_out, pre)
    T, d = x.shape
    E, inter = routed["w1"].shape[0], routed["w1"].shape[1]
    rows = T * k + (T if shared is not None else 0)
    dx_rows = torch.empty(rows, d, dtype=torch.float32, device=x.device) if dx_rows is None else dx_rows
    gl = lambda b: {n: torch.empty(b[n].shape[:-1] + (d if n != "w2" else inter,), dtype=torch.float32,  # noqa: E731
                                   device=x.device) for n in ("w1", "w3", "w2")}
    grads = gl(routed) if grads is None else grads
    if shared is not None and shared_grads is None:
        shared_grads = gl(shared)
    rb, sb = _bank(routed), _bank(shared)
    rt, st = _tbank(routed_t), _tbank(shared_t)
    rg, sg = _grads(grads), _grads(shared_grads)
    ref = lambda v: ctypes.byref(v) if v is not None else None  # noqa: E731
    _ok(lib().moe_expert_ffn_backward_nvfp4(_ptr(x), T, d, E, k, inter, ref(rb), ref(sb), ref(rt), ref(st),
                                            _ptr(offsets), _ptr(perm), _ptr(pre), _ptr(d_out), _ptr(dx_rows),
                                            ref(rg), ref(sg), ws.ptr, ws.nbytes, _stream(x.device)),
        "moe_expert_ffn_backward_nvfp4")
    return dx_rows, grads, shared_grads


def moe_nvfp4_pack_weights(codes, block_scales):
    """K-blocked copy of NVFP4 weight matrices: codes [n][R][K/2] and block scales
    [n][R][K/16] (or one matrix without the leading n) -> (packed codes, packed scales),
    the layout an NVFP4 expert bank takes."""
    _check_dev(codes, block_scales)
    shape = codes.shape
    c = codes.reshape(-1, shape[-2], shape[-1]).contiguous()
    sc = block_scales.reshape(-1, shape[-2], block_scales.shape[-1]).contiguous()
    n, R, K = c.shape[0], c.shape[1], c.shape[2] * 2
    if sc.shape != (n, R, K // 16):
        raise ValueError(f"block scales {tuple(block_scales.shape)} do not match codes {tuple(shape)}")
    pc, ps = torch.empty_like(c), torch.empty_like(sc)
    _ok(lib().moe_nvfp4_pack_weights(_ptr(c), _ptr(sc), n, R, K, _ptr(pc), _ptr(ps), _stream(c.device)),
        "moe_nvfp4_pack_weights")
    return pc.reshape(shape), ps.reshape(block_scales.shape)


def nvfp4_pack_inputs(inp):
    """A copy of a layer's input dict whose NVFP4 expert weights (row-major codes and
    block scales, routed and shared) are K-blocked for the expert FFN."""
    out = dict(inp)

    def pack(b):
        b = dict(b)
        for n in ("w1", "w3", "w2"):
            b[n], b[n + "_scale"] = moe_nvfp4_pack_weights(b[n], b[n + "_scale"])
        return b

    out.update({kk: vv for kk, vv in pack({n: inp[n] for n in ("w1", "w3", "w2", "w1_scale", "w3_scale",
                                                               "w2_scale")}).items()})
    if inp.get("shared") is not None:
        out["shared"] = pack(inp["shared"])
    return out


def moe_nvfp4_quantize(x, codes=None, block_scales=None, row_scales=None):
    """NVFP4 rows of a bf16 matrix: (codes [R][K/2] uint8, block scales [R][K/16] uint8,
    row scales [R] fp32)."""
    _check_dev(x)
    R, K = x.shape
    dev = x.device
    codes = torch.empty(R, K // 2, dtype=torch.uint8, device=dev) if codes is None else codes
    block_scales = torch.empty(R, K // 16, dtype=torch.uint8, device=dev) if block_scales is None else block_scales
    row_scales = torch.empty(R, dtype=torch.float32, device=dev) if row_scales is None else row_scales
    _ok(lib().moe_nvfp4_quantize(_ptr(x), R, K, _ptr(codes), _ptr(block_scales), _ptr(row_scales),
                                 _stream(dev)), "moe_nvfp4_quantize")
    return codes, block_scales, row_scales
