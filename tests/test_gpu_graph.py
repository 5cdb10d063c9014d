"""The verify step captured in a HIP graph and replayed.

A call only enqueues kernels on the caller's stream (no allocation, no
synchronisation, no memset), so a serving loop can capture it once and replay
it.  Each case captures one call with preallocated outputs and workspace,
replays it several times with eager work and synchronisations in between,
and checks every replay against an eager call, also after new uniforms are
written into the captured input buffers.
"""
import dataclasses
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

CASES = {
    "small-16": lambda: workloads.make_batch(1, seqs=range(16)),
    "headline-16-split": lambda: workloads.make_batch(2, seqs=range(16), workers=workloads.default_workers()),
    "small-160": lambda: workloads.make_batch(1, seqs=range(160), workers=workloads.default_workers()),
    "short-rows-48": lambda: workloads.make_batch(0, seqs=range(48)),  # one launch (k_short)
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("ragged", [False, True], ids=["full", "ragged"])
def test_graph_replays_match_eager(gpu_lib, name, ragged):
    import torch
    sv = gpu_lib
    b = CASES[name]()
    lp, lq, x, ua, ur = workloads.to_device(b)
    B, K, V, T = b.B, b.K, b.V, b.T
    dt = sv.SPECV_BF16 if b.dtype == "bf16" else sv.SPECV_F32
    ws = torch.empty(sv.workspace_size(B, K, V, dt, T), dtype=torch.uint8, device="cuda")
    tok = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    n = torch.empty((B,), dtype=torch.int32, device="cuda")
    kb = torch.from_numpy(workloads.ragged_draft_counts(B, K, seed=3, low=0)).cuda() if ragged else None
    print(f"[graph] {name} {'ragged' if ragged else 'full'}: {b.wl.describe()}", file=sys.stderr, flush=True)

    def call():
        rc = (sv.spec_verify_ragged(lp, lq, x, kb, ua, ur, T, tok, n, ws) if ragged
              else sv.spec_verify(lp, lq, x, ua, ur, T, tok, n, ws))
        assert rc == 0, sv.strerror(rc)

    def eager():
        call()
        torch.cuda.synchronize()
        return tok.clone(), n.clone()

    ref = eager()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    rng = np.random.default_rng(11)
    for rep in range(4):
        if rep == 2:  # new uniforms in the captured buffers: the replay must use them
            ua.copy_(torch.from_numpy(workloads.uniforms(rng, B * K).reshape(B, K)).cuda())
            ur.copy_(torch.from_numpy(workloads.uniforms(rng, B)).cuda())
            ref = eager()
        tok.fill_(-7)
        n.fill_(-7)
        _ = torch.ones(1 << 16, device="cuda").cumsum(0)  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(n.cpu().numpy(), ref[1].cpu().numpy(), err_msg=f"replay {rep}")
        np.testing.assert_array_equal(tok.cpu().numpy(), ref[0].cpu().numpy(), err_msg=f"replay {rep}")
