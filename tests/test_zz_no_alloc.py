"""spec_verify_noalloc (the entry point for callers that cannot allocate)
against spec_verify, through the C ABI: the same kernels on a static scratch
instead of a caller's workspace must give the same outputs, call after call,
also when a call follows a larger one (the scratch keeps the previous call's
contents), and both must match the fp64 oracle."""
import ctypes
import sys

import numpy as np
import pytest

import oracle
import workloads
from oracle.parity import GpuOut, compare

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _both(sv, batch):
    """(spec_verify outputs, spec_verify_noalloc outputs) on one batch, as
    host arrays; the noalloc outputs start as a sentinel so unwritten entries show."""
    import torch
    lib = sv.load()
    lp, lq, x, ua, ur = workloads.to_device(batch)
    B, K, V, T = batch.B, batch.K, batch.V, batch.T
    dt = sv.SPECV_BF16 if batch.dtype == "bf16" else sv.SPECV_F32
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    need = sv.workspace_size(B, K, V, dt, T)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    t1 = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    n1 = torch.empty((B,), dtype=torch.int32, device="cuda")
    t2 = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
    n2 = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    args = (_ptr(lp), _ptr(lq), _ptr(x), _ptr(ua), _ptr(ur), ctypes.c_float(T), B, K, V)
    assert lib.spec_verify(*args, _ptr(t1), _ptr(n1), dt, _ptr(ws), ctypes.c_size_t(need), st) == 0
    assert lib.spec_verify_noalloc(*args, _ptr(t2), _ptr(n2), dt, st) == 0
    torch.cuda.synchronize()
    return (t1.cpu().numpy(), n1.cpu().numpy()), (t2.cpu().numpy(), n2.cpu().numpy())


def _check(sv, batch, label):
    (t1, n1), (t2, n2) = _both(sv, batch)
    np.testing.assert_array_equal(t2, t1, err_msg=label)
    np.testing.assert_array_equal(n2, n1, err_msg=label)
    ref = oracle.verify_batch(batch, workers=workloads.default_workers())
    rep = compare(batch, GpuOut(t2, n2, None, None), ref)
    say(f"[noalloc] {label}: {batch.wl.describe()} decisions={rep.decisions} excused={rep.excused}")
    rep.check()


def test_noalloc_matches_spec_verify_larger_then_smaller(gpu_lib):
    """Two calls in a row, the second smaller: the headline shape at full
    size (one workgroup per sequence in the draw), then 48 of its sequences
    (the split draw, whose counters and published sums live in the scratch),
    then the small workload; greedy in between."""
    _check(gpu_lib, workloads.make_batch(2, workers=workloads.default_workers()), "headline B=256")
    _check(gpu_lib, workloads.make_batch(2, seqs=range(48), workers=workloads.default_workers()), "headline B=48")
    _check(gpu_lib, workloads.make_batch(4, seqs=range(40), workers=workloads.default_workers()), "greedy B=40")
    _check(gpu_lib, workloads.make_batch(1, seqs=range(16), workers=workloads.default_workers()), "small B=16")
    _check(gpu_lib, workloads.make_batch(0), "tiny B=1")


def test_noalloc_rejects_a_shape_beyond_its_scratch(gpu_lib):
    """A shape that needs more than the scratch returns SPECV_E_SCRATCH and
    enqueues nothing: the outputs keep their sentinel."""
    import torch
    lib = gpu_lib.load()
    B, K, V = 4096, 4, 256000
    assert gpu_lib.workspace_size(B, K, V, gpu_lib.SPECV_F32, 1.0) > gpu_lib.NOALLOC_SCRATCH
    small = torch.zeros(16, dtype=torch.float32, device="cuda")  # never read: the call stops on the host
    t = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    rc = lib.spec_verify_noalloc(_ptr(small), _ptr(small), _ptr(t), _ptr(small), _ptr(small), ctypes.c_float(1.0),
                                 B, K, V, _ptr(t), _ptr(t), gpu_lib.SPECV_F32,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == -8
    assert torch.all(t == -7)
