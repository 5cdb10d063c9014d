"""spec_verify_sweep_timed: an event pair recorded with each row-sweep launch
(the benchmark's per-kernel roofline).  With the rounds on (the tests'
threshold is 0) a K=5 call has three sweep launches, a call that asks for
log Z one; every pair times a launch of positive length, the launches fit
inside the span from the first start to the last end, and the outputs are
spec_verify_ex's."""
import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


class _Events:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.begin, self.end = [], []
        for lst in (self.begin, self.end):
            for _ in range(n):
                e = ctypes.c_void_p()
                assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
                lst.append(e.value)

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value

    def close(self):
        for e in self.begin + self.end:
            self.hip.hipEventDestroy(e)


def test_each_sweep_launch_is_timed(gpu_lib):
    sv = gpu_lib
    b = workloads.make_batch(1, seqs=range(64))
    lp, lq, x, ua, ur = workloads.to_device(b)
    B, K, V, T = b.B, b.K, b.V, b.T
    ws = torch.empty(sv.workspace_size(B, K, V, sv.SPECV_BF16, T), dtype=torch.uint8, device="cuda")

    def outputs():
        return (torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda"),
                torch.full((B,), -7, dtype=torch.int32, device="cuda"),
                torch.full((B,), -7, dtype=torch.int32, device="cuda"))

    rt, rn, rf = outputs()
    assert sv.spec_verify(lp, lq, x, ua, ur, T, rt, rn, ws, out_flags=rf, extended=True) == 0
    ev = _Events(3)
    try:
        t, n, f = outputs()
        rc, ns = sv.spec_verify_sweep_timed(lp, lq, x, ua, ur, T, t, n, ws, ev.begin, ev.end, out_flags=f)
        torch.cuda.synchronize()
        assert rc == 0 and ns == 3, (rc, ns)
        launches = [ev.ms(ev.begin[i], ev.end[i]) for i in range(3)]
        span = ev.ms(ev.begin[0], ev.end[2])
        print(f"[timing] sweep launches {launches} ms, phase {span} ms", flush=True)
        assert all(v > 0 for v in launches) and sum(launches) <= span
        for got, ref in ((t, rt), (n, rn), (f, rf)):
            np.testing.assert_array_equal(got.cpu().numpy(), ref.cpu().numpy())
        # every row in one sweep when log Z is asked for: one launch, timed by the first pair
        logz = torch.empty((B, 2 * K + 1), dtype=torch.float32, device="cuda")
        t, n, f = outputs()
        rc, ns = sv.spec_verify_sweep_timed(lp, lq, x, ua, ur, T, t, n, ws, ev.begin, ev.end, out_logz=logz,
                                            out_flags=f)
        torch.cuda.synchronize()
        assert rc == 0 and ns == 1 and ev.ms(ev.begin[0], ev.end[0]) > 0
        np.testing.assert_array_equal(t.cpu().numpy(), rt.cpu().numpy())
        # no events: the count is still reported
        rc, ns = sv.spec_verify_sweep_timed(lp, lq, x, ua, ur, T, t, n, ws, [], [])
        torch.cuda.synchronize()
        assert rc == 0 and ns == 3
    finally:
        ev.close()


def test_short_rows_one_launch_is_timed(gpu_lib):
    """Rows of at most 2048 tokens take one launch for the whole step: the
    timed entry point reports one launch, times it with the first pair, and
    gives spec_verify_ex's outputs."""
    sv = gpu_lib
    b = workloads.make_batch(0, seqs=range(16))
    lp, lq, x, ua, ur = workloads.to_device(b)
    B, K, V, T = b.B, b.K, b.V, b.T
    ws = torch.empty(sv.workspace_size(B, K, V, sv.SPECV_F32, T), dtype=torch.uint8, device="cuda")
    rt = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
    rn = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    rf = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    assert sv.spec_verify(lp, lq, x, ua, ur, T, rt, rn, ws, out_flags=rf, extended=True) == 0
    ev = _Events(3)
    try:
        t, n, f = torch.empty_like(rt), torch.empty_like(rn), torch.empty_like(rf)
        rc, ns = sv.spec_verify_sweep_timed(lp, lq, x, ua, ur, T, t, n, ws, ev.begin, ev.end, out_flags=f)
        torch.cuda.synchronize()
        assert rc == 0 and ns == 1, (rc, ns)
        assert ev.ms(ev.begin[0], ev.end[0]) > 0
        for got, ref in ((t, rt), (n, rn), (f, rf)):
            np.testing.assert_array_equal(got.cpu().numpy(), ref.cpu().numpy())
        assert np.all(f.cpu().numpy() & sv.FLAG_FP64)
    finally:
        ev.close()
