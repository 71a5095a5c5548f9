"""The C-ABI library on the CPU: it loads, exports every call include/moe.h declares,
and rejects invalid arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

import parity_gate_gemm_amd as pg
from parity_gate_gemm_amd import build as pg_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every case returns before a launch


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pg.LIB_PATH):
        pg_build.build()
    return pg.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"moe_route", "moe_route_replay", "moe_dispatch", "moe_expert_ffn", "moe_combine"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(7):
        assert pg.moe_status_string(code).startswith("MOE_")
    assert "unknown" in pg.moe_status_string(99)


def test_workspace_size(L):
    a = pg.moe_workspace_size(4096, 7168, 384, 8, 2048, pg.MOE_BF16)
    b = pg.moe_workspace_size(32, 128, 384, 8, 64, pg.MOE_F32)
    assert a > 4096 * 384 * 8 and a > (4096 * 9) * 2048 * 2
    assert b > 0
    assert pg.moe_workspace_size(0, 128, 16, 2, 64, pg.MOE_BF16) > 0
    assert pg.moe_workspace_size(0, 64, 16, 2, 64, pg.MOE_BF16) > 0      # empty batch, short rows
    assert pg.moe_workspace_size(0, 7168, 384, 8, 2048, pg.MOE_MXFP8) > 0
    n = ctypes.c_size_t()
    for bad in [(-1, 128, 16, 2, 64, 1), (8, 0, 16, 2, 64, 1), (8, 128, 2000, 2, 64, 1),
                (8, 128, 16, 17, 64, 1), (8, 128, 16, 33, 64, 1), (8, 128, 64, 33, 64, 1),
                (8, 128, 16, 2, 0, 1), (8, 128, 16, 2, 64, 7)]:
        assert L.moe_workspace_size(*bad, ctypes.byref(n)) == 1, bad
    assert L.moe_workspace_size(8, 128, 16, 2, 64, 1, None) == 1


def test_route_host_validation(L):
    P = FAKE
    # T == 0 is a no-op
    assert L.moe_route(None, None, 1, 0, 128, None, None, 16, 2, None, None, None, 0, None) == 0
    assert L.moe_route(None, None, 1, 4, 128, P, None, 16, 2, P, P, P, 1 << 30, None) == 1   # null x
    assert L.moe_route(P, None, 1, 4, 128, P, None, 2000, 2, P, P, P, 1 << 30, None) == 1    # E too big
    assert L.moe_route(P, None, 1, 4, 128, P, None, 16, 0, P, P, P, 1 << 30, None) == 1      # k = 0
    assert L.moe_route(P, None, 9, 4, 128, P, None, 16, 2, P, P, P, 1 << 30, None) == 1      # dtype
    assert L.moe_route(P, None, 2, 4, 128, P, None, 16, 2, P, P, P, 1 << 30, None) == 1      # MXFP8 w/o scale
    assert L.moe_route(P, P, 2, 4, 100, P, None, 16, 2, P, P, P, 1 << 30, None) == 1         # d % 32
    assert L.moe_route(P, P, 1, 4, 128, P, None, 16, 2, P, P, P, 1 << 30, None) == 1         # scale w/ bf16
    assert L.moe_route(P, None, 1, 4, 128, P, None, 16, 2, P, P, P, 64, None) == 3           # workspace
    assert L.moe_route(P, None, 1, 4, 128, P, None, 16, 2, None, P, P, 1 << 30, None) == 1   # null ids
    assert L.moe_route_replay(P, None, 1, 4, 128, P, None, 16, 2, None, None, P, P, 1 << 30, None) == 1
    F, Q = L.moe_route_replay_filtered, ctypes.c_void_p(0x20000)
    assert F(None, None, 1, 0, 128, None, None, 16, 2, None, 0.0, None, None, None, 0, None) == 0
    assert F(P, None, 1, 4, 128, P, None, 16, 2, P, float("nan"), Q, P, P, 1 << 30, None) == 1  # NaN tau
    assert F(P, None, 1, 4, 128, P, None, 16, 2, P, 0.0, ctypes.c_void_p(0x10008), P, P, 1 << 30,
             None) == 1                                                                        # overlap
    assert F(P, None, 1, 4, 128, P, None, 16, 2, P, 0.0, None, P, P, 1 << 30, None) == 1       # null ids_out
    assert F(P, None, 1, 4, 128, P, None, 16, 2, None, 0.0, Q, P, P, 1 << 30, None) == 1       # null ids_in
    assert F(P, None, 1, 4, 128, P, None, 16, 2, P, 0.0, Q, P, P, 64, None) == 3               # workspace


def test_dispatch_ffn_combine_host_validation(L):
    P = FAKE
    assert L.moe_dispatch(P, 4, 0, 2, P, P, P, P, 1 << 30, None) == 1
    assert L.moe_dispatch(P, 4, 16, 40, P, P, P, P, 1 << 30, None) == 1
    assert L.moe_dispatch(P, 4, 16, 2, P, P, P, P, 16, None) == 3
    assert L.moe_dispatch(None, 4, 16, 2, P, P, P, P, 1 << 30, None) == 1
    bank = pg._Bank(0x10000, 0x10000, 0x10000, None, None, None)
    nob = pg._Bank(0x10000, None, 0x10000, None, None, None)
    B = ctypes.byref(bank)
    assert L.moe_expert_ffn(P, None, 1, 4, 128, 16, 2, 64, ctypes.byref(nob), None, P, P, P, P, 1 << 30, None) == 1
    assert L.moe_expert_ffn(P, None, 1, 4, 96, 16, 2, 64, B, None, P, P, P, P, 1 << 30, None) == 2   # d % 128
    assert L.moe_expert_ffn(P, None, 1, 4, 128, 16, 2, 48, B, None, P, P, P, P, 1 << 30, None) == 2  # I % 64
    assert L.moe_expert_ffn(P, None, 1, 4, 128, 16, 2, 64, B, None, P, P, P, P, 64, None) == 3
    sbank = pg._Bank(0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000)
    assert L.moe_expert_ffn(P, P, 2, 4, 128, 16, 2, 64, ctypes.byref(sbank), None, P, P, P, P, 1 << 30, None) == 2
    assert L.moe_expert_ffn(P, None, 1, 0, 128, 16, 2, 64, B, None, P, None, None, P, 1 << 30, None) == 0
    assert L.moe_combine(P, 1, P, P, 4, 100, 2, 0, P, None) == 2
    assert L.moe_combine(P, 1, P, P, 4, 128, 0, 0, P, None) == 1
    assert L.moe_combine(None, 1, P, P, 4, 128, 2, 0, P, None) == 1
    assert L.moe_combine(P, 1, P, P, 0, 128, 2, 0, P, None) == 0
    # backward calls
    G = pg._GradBank(0x10000, 0x10000, 0x10000)
    GB = ctypes.byref(G)
    assert L.moe_combine_backward(P, 1, P, P, P, 4, 100, 2, 0, P, P, None) == 2           # d % 8
    assert L.moe_combine_backward(None, 1, P, P, P, 4, 128, 2, 0, P, P, None) == 1
    assert L.moe_combine_backward(P, 1, P, P, P, 0, 128, 2, 0, P, P, None) == 0           # T = 0
    assert L.moe_expert_ffn_backward(P, None, 0, 4, 128, 16, 2, 128, B, None, P, P, None, P, P, GB,
                                     None, P, 1 << 30, None) == 2                          # fp32
    assert L.moe_expert_ffn_backward(P, None, 1, 4, 128, 16, 2, 64, B, None, P, P, None, P, P, GB,
                                     None, P, 1 << 30, None) == 2                          # I % 128
    assert L.moe_expert_ffn_backward(P, None, 1, 4, 128, 16, 2, 128, B, B, P, P, None, P, P, GB,
                                     None, P, 1 << 30, None) == 1                          # shared w/o grads
    assert L.moe_expert_ffn_backward(P, None, 1, 4, 128, 16, 2, 128, B, None, P, P, None, P, P, GB,
                                     None, P, 64, None) == 3                               # workspace
    assert L.moe_expert_ffn_backward(P, None, 1, 4, 128, 16, 2, 128, B, None, P, P,
                                     ctypes.c_void_p(0x10008), P, P, GB, None, P, 1 << 30, None) == 1
    assert L.moe_expert_ffn_gate_up_save(P, None, 2, 4, 128, 16, 2, 128, B, None, P, P, P, P,
                                         1 << 30, None) in (1, 2)                          # mxfp8
    assert L.moe_route_backward(P, None, 1, 4, 128, P, 16, 2, P, P, P, P, P, P, P, 0, P, None, P,
                                P, 1 << 30, None) == 1                                     # bias w/o gate
    assert L.moe_route_backward(P, None, 1, 4, 126, P, 16, 2, P, P, P, P, P, P, P, 0, P, P, None,
                                P, 1 << 30, None) == 2                                     # d % 4
    assert L.moe_route_backward(P, None, 1, 4, 128, P, 16, 2, P, P, P, P, P, P, P, 0, P, P, None,
                                P, 64, None) == 3                                          # workspace
    n = ctypes.c_size_t()
    assert L.moe_backward_workspace_size(4096, 7168, 384, 8, 2048, 1, ctypes.byref(n)) == 0
    assert n.value >= pg.moe_workspace_size(4096, 7168, 384, 8, 2048, 1)
    assert L.moe_check(None, 0, None) == 1
    assert L.moe_workspace_init(None, 0, None) == 1


def test_nvfp4_host_validation(L):
    P = FAKE
    A = ctypes.c_void_p(0x20000)          # a second, disjoint fake range
    # quantizer: bad K, nulls, misalignment; rows == 0 is a no-op
    assert L.moe_nvfp4_quantize(P, 4, 24, P, P, P, None) == 1
    assert L.moe_nvfp4_quantize(P, 4, 32, None, P, P, None) == 1
    assert L.moe_nvfp4_quantize(ctypes.c_void_p(0x10008), 4, 32, A, P, P, None) == 1
    assert L.moe_nvfp4_quantize(None, 0, 32, None, None, None, None) == 0
    # K-blocking: R % 32, K % 64, nulls, alignment, overlap; empty is a no-op
    big = ctypes.c_void_p(0x100000)
    assert L.moe_nvfp4_pack_weights(P, A, 1, 48, 64, big, ctypes.c_void_p(0x200000), None) == 1
    assert L.moe_nvfp4_pack_weights(P, A, 1, 32, 96, big, ctypes.c_void_p(0x200000), None) == 1
    assert L.moe_nvfp4_pack_weights(P, None, 1, 32, 64, big, ctypes.c_void_p(0x200000), None) == 1
    assert L.moe_nvfp4_pack_weights(ctypes.c_void_p(0x10004), A, 1, 32, 64, big,
                                    ctypes.c_void_p(0x200000), None) == 1
    assert L.moe_nvfp4_pack_weights(P, A, 1, 32, 64, P, ctypes.c_void_p(0x200000), None) == 1   # in place
    assert L.moe_nvfp4_pack_weights(P, A, 1, 32, 64, big, big, None) == 1                     # outputs overlap
    assert L.moe_nvfp4_pack_weights(None, None, 0, 32, 64, None, None, None) == 0
    assert L.moe_nvfp4_pack_weights(P, A, -1, 32, 64, big, big, None) == 1
