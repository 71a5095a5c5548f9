"""moe_dispatch_noalloc (the dispatch entry point with its scratch in a static device
array) against moe_dispatch (workspace scratch) and the oracle's dispatch: bit-exact
offsets, perm and row_of on consecutive calls of decreasing size, the device status on
bad ids, and the host-side size limit."""
import numpy as np
import pytest
import torch

import oracle
import parity_gate_gemm_amd as pg
import synth
from _gpu_common import say

pytestmark = pytest.mark.gpu


def _both(ids, E):
    T, k = ids.shape
    ws = pg.Workspace(T, 64, E, k, 64, pg.MOE_BF16)
    ref = pg.moe_dispatch(ids, E, ws)
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    got = pg.moe_dispatch_noalloc(ids, E, status=st)
    torch.cuda.synchronize()
    return ref, got, int(st.item()), pg.moe_check(ws)


def test_noalloc_dispatch_matches_workspace_dispatch():
    rng = np.random.Generator(np.random.PCG64(7))
    cases = [(32768, 384, 8), (4096, 384, 8), (700, 384, 8), (1, 16, 3)]   # decreasing sizes
    for T, E, k in cases:
        say(f"case noalloc dispatch T={T} E={E} k={k}")
        ids_np = synth.zipf_replay_ids(T, E, k, 1.2, rng)
        ids = torch.from_numpy(ids_np).cuda()
        ref, got, st, st_ws = _both(ids, E)
        assert st == 0 and st_ws == 0
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        o, p, r = oracle.dispatch(ids_np, E)
        assert np.array_equal(got[0].cpu().numpy(), o)
        assert np.array_equal(got[1].cpu().numpy(), p)
        assert np.array_equal(got[2].cpu().numpy(), r)


def test_noalloc_dispatch_bad_ids_status_and_clear():
    rng = np.random.Generator(np.random.PCG64(8))
    E, k = 64, 4
    ids_np = synth.zipf_replay_ids(300, E, k, 1.2, rng)
    bad = ids_np.copy()
    bad[17, 2] = E                      # out of range: flagged, counted as expert 0
    say("case noalloc dispatch with an out-of-range id")
    ref, got, st, st_ws = _both(torch.from_numpy(bad).cuda(), E)
    assert st == 4 and st_ws == 4       # MOE_ERR_BAD_IDS from both entry points
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    say("case noalloc dispatch after the bad call: status cleared")
    ref, got, st, st_ws = _both(torch.from_numpy(ids_np[:100].copy()).cuda(), E)
    assert st == 0 and st_ws == 0
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_noalloc_dispatch_empty_and_size_limit():
    say("case noalloc dispatch empty batch and size limit")
    ids = torch.empty(0, 2, dtype=torch.int32, device="cuda")
    off, _, _ = pg.moe_dispatch_noalloc(ids, 16)
    torch.cuda.synchronize()
    assert torch.all(off == 0)
    # 4 MiB of scratch holds ceil(T / 64) + 1 histogram rows of E ints after 256 bytes
    big = 64 * ((4 * 2 ** 20 - 256) // (4 * 1024))     # one block row more than fits at E = 1024
    assert pg.lib().moe_dispatch_noalloc(None, big, 1024, 1, pg._ptr(off), None, None, None, None) == 2
