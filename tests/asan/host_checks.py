"""Host-side argument checks of libspecverify, run against a CPU
AddressSanitizer build of api.cpp (tests/test_asan_host.py builds it and runs
this file in a subprocess with libasan preloaded; no torch, no GPU).

usage: python host_checks.py LIB.so"""
import ctypes
import sys

lib = ctypes.CDLL(sys.argv[1])
vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
common = [vp, vp, vp, vp, vp, f32, i32, i32, i32, vp, vp, i32, vp, sz, vp]
sigs = {
    "spec_verify_workspace_size": ([i32, i32, i32, i32, f32], sz),
    "spec_verify": (common, i32),
    "spec_verify_ex": (common + [vp] * 4, i32),
    "spec_verify_noalloc": (common[:12] + [vp], i32),
    "spec_verify_sweep_timed": (common + [vp] * 4 + [i32, vp], i32),
    "spec_verify_ragged": ([vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, vp, vp, vp, i32, vp, sz, vp], i32),
    "spec_verify_ragged_ex": ([vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, vp, vp, vp, i32, vp, sz, vp, vp, vp], i32),
    "spec_verify_tree_workspace_size": ([i32] * 4, sz),
    "spec_verify_tree_greedy": ([vp, vp, vp, i32, i32, i32, vp, vp, vp, i32, vp, sz, vp], i32),
    "spec_tree_mask": ([vp, i32, i32, vp, vp, vp], i32),
    "spec_ngram_propose": ([vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp], i32),
    "spec_ngram_map_bytes": ([i32, i32], sz),
    "spec_rounds_min_bytes": ([ctypes.c_double], ctypes.c_double),
    "spec_short_max_seqs": ([ctypes.c_int], ctypes.c_int),
    "spec_ngram_map_update": ([vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp], i32),
    "spec_verify_strerror": ([i32], ctypes.c_char_p),
    "spec_verify_version": ([], ctypes.c_char_p),
    "spec_debug_enable": ([i32], i32),
    "spec_debug_counters": ([vp, i32], i32),
    "spec_debug_reset": ([], i32),
}
for name, (args, res) in sigs.items():
    f = getattr(lib, name)
    f.argtypes, f.restype = args, res

F32, BF16 = 0, 1
P, Q, X, UA, UR, OT, ON, KB, LZ, FL = (0x10000 * i for i in range(1, 11))
WS = 0x7000000
BIG = 1 << 30

# workspace sizes, including shapes at the edges of the checks
assert lib.spec_verify_workspace_size(256, 8, 128256, BF16, 0.7) > 0
assert lib.spec_verify_workspace_size(1024, 4, 256000, F32, 1.0) > 0
for bad in [(0, 8, 100, BF16, 1.0), (4, 0, 100, BF16, 1.0), (4, 33, 100, BF16, 1.0), (4, 8, 0, BF16, 1.0),
            (4, 8, 100, 7, 1.0), (4, 8, 100, BF16, -1.0), (4, 8, 100, BF16, float("nan")),
            (4, 8, 100, BF16, float("inf")), (4, 8, 100, BF16, 1e-45), (1 << 30, 32, 1 << 30, F32, 1.0)]:
    assert lib.spec_verify_workspace_size(*bad) == 0, bad

v = lambda *a, **k: lib.spec_verify(*a)
assert lib.spec_verify(None, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, WS, BIG, None) == -1
assert lib.spec_verify(P, None, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, WS, BIG, None) == -1
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 4, 3, 128, None, ON, F32, WS, BIG, None) == -1
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, 5, WS, BIG, None) == -3
assert lib.spec_verify(P, Q, X, UA, UR, float("nan"), 4, 3, 128, OT, ON, F32, WS, BIG, None) == -4
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 0, 3, 128, OT, ON, F32, WS, BIG, None) == -2
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 4, 33, 128, OT, ON, F32, WS, BIG, None) == -2
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 4, 3, 0, OT, ON, F32, WS, BIG, None) == -2
assert lib.spec_verify(P + 2, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, WS, BIG, None) == -6
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, None, BIG, None) == -5
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, WS + 8, BIG, None) == -5
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, WS, 16, None) == -5
# valid arguments reach the (stubbed) launches: sampling, greedy, unaligned rows, both sweep paths
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, WS, BIG, None) == -7
assert lib.spec_verify(P, None, X, None, None, 0.0, 4, 3, 128, OT, ON, BF16, WS, BIG, None) == -7
assert lib.spec_verify(P + 4, Q + 4, X, UA, UR, 0.5, 4, 3, 127, OT, ON, F32, WS, BIG, None) == -7
assert lib.spec_verify(P, Q, X, UA, UR, 0.7, 4096, 8, 128256, OT, ON, BF16, WS, 1 << 40, None) == -7
assert lib.spec_verify_ex(P, Q, X, UA, UR, 0.7, 4096, 8, 128256, OT, ON, BF16, WS, 1 << 40, None, LZ, FL,
                          None, None) == -7
assert lib.spec_verify_ex(P, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, 9, WS, BIG, None, LZ, FL, None, None) == -3
# ragged and ragged_ex
assert lib.spec_verify_ragged(P, Q, X, None, UA, UR, 1.0, 4, 3, 128, OT, ON, None, F32, WS, BIG, None) == -1
assert lib.spec_verify_ragged(P, Q, X, KB, UA, UR, 1.0, 4, 3, 128, OT, ON, None, F32, WS, 16, None) == -5
assert lib.spec_verify_ragged(P, Q, X, KB, UA, UR, 1.0, 4, 3, 128, OT, ON, None, F32, WS, BIG, None) == -7
assert lib.spec_verify_ragged_ex(P, Q, X, KB, UA, UR, 1.0, 4, 3, 128, OT, ON, None, F32, WS, BIG, None, LZ,
                                 FL) == -7
assert lib.spec_verify_ragged_ex(P + 2, Q, X, KB, UA, UR, 1.0, 4, 3, 128, OT, ON, None, F32, WS, BIG, None, LZ,
                                 FL) == -6
# no-allocation entry point: argument errors, the scratch limit, then the (stubbed) symbol lookup
assert lib.spec_verify_noalloc(None, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, None) == -1
assert lib.spec_verify_noalloc(P, Q, X, UA, UR, 1.0, 4096, 4, 256000, OT, ON, F32, None) == -8
assert lib.spec_verify_noalloc(P, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, None) == -7
# trees, tree mask, n-gram proposer
L, TT, PA, OTT, OP, ONN = (0x100000 * i for i in range(1, 7))
assert lib.spec_verify_tree_workspace_size(4, 16, 1000, BF16) > 0
assert lib.spec_verify_tree_workspace_size(4, 65, 1000, BF16) == 0
assert lib.spec_verify_tree_greedy(L, TT, PA, 4, 16, 1000, OTT, OP, ONN, BF16, WS, 64, None) == -5
assert lib.spec_verify_tree_greedy(L + 1, TT, PA, 4, 16, 1000, OTT, OP, ONN, BF16, WS, BIG, None) == -6
assert lib.spec_verify_tree_greedy(L, TT, PA, 4, 16, 1000, OTT, OP, ONN, BF16, WS, BIG, None) == -7
assert lib.spec_tree_mask(PA, 4, 65, OTT, OP, None) == -2
assert lib.spec_tree_mask(PA, 4, 16, OTT, OP, None) == -7
assert lib.spec_ngram_propose(L, TT, 4, 100, 3, 2, 1, 5, OTT, OP, None) == -2
assert lib.spec_ngram_propose(L, TT, 4, 100, 1, 4, 1, 5, OTT, OP, None) == -7
assert lib.spec_ngram_map_bytes(4, 1024) == 4 * (16 + 16 * 1024) and lib.spec_ngram_map_bytes(4, 1000) == 0
old = lib.spec_rounds_min_bytes(-1.0)
assert lib.spec_rounds_min_bytes(12345.0) == old and lib.spec_rounds_min_bytes(float("nan")) == 12345.0
assert lib.spec_rounds_min_bytes(old) == 12345.0
old = lib.spec_short_max_seqs(-1)
assert lib.spec_short_max_seqs(5) == old and lib.spec_short_max_seqs(-1) == 5 and lib.spec_short_max_seqs(old) == 5
assert lib.spec_ngram_map_update(WS, 1024, L, TT, PA, 4, 100, 3, 2, 1, 5, OTT, OP, None, None) == -2
assert lib.spec_ngram_map_update(WS + 8, 1024, L, TT, PA, 4, 100, 1, 4, 1, 5, OTT, OP, None, None) == -6
assert lib.spec_ngram_map_update(WS, 1024, L, TT, PA, 4, 100, 1, 4, 1, 5, OTT, OP, None, None) == -7
# per-launch sweep timing: its own checks, then the common ones; the number
# of launches is written on every return
NS = ctypes.c_int(7)
EVB = (vp * 3)(0x100, 0x200, 0x300)
EVE = (vp * 3)(0x101, 0x201, 0x301)
T3 = (P, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, WS, BIG, None, None, None)
assert lib.spec_verify_sweep_timed(*T3, ctypes.cast(EVB, vp), ctypes.cast(EVE, vp), -1, ctypes.byref(NS)) == -2
assert NS.value == 0
assert lib.spec_verify_sweep_timed(*T3, None, ctypes.cast(EVE, vp), 3, ctypes.byref(NS)) == -1
assert lib.spec_verify_sweep_timed(*T3[:4], None, *T3[5:], ctypes.cast(EVB, vp), ctypes.cast(EVE, vp), 3,
                                   ctypes.byref(NS)) == -1
assert lib.spec_verify_sweep_timed(*T3, ctypes.cast(EVB, vp), ctypes.cast(EVE, vp), 3, None) == -7
assert lib.spec_verify_sweep_timed(*T3, None, None, 0, ctypes.byref(NS)) == -7

# device-side validation: argument checks, the HIP errors of the stand-ins,
# and a verify call with validation on (its validation launch fails first)
CNT = (ctypes.c_ulonglong * 8)()
assert lib.spec_debug_counters(None, 1) == -1
assert lib.spec_debug_counters(ctypes.cast(CNT, vp), 0) == -2
assert lib.spec_debug_counters(ctypes.cast(CNT, vp), 8) == -2
assert lib.spec_debug_counters(ctypes.cast(CNT, vp), 7) == -7
assert lib.spec_debug_reset() == -7
assert lib.spec_debug_enable(1) == 0
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 4, 3, 128, OT, ON, F32, WS, BIG, None) == -7
assert lib.spec_verify(P, Q, X, UA, UR, 1.0, 0, 3, 128, OT, ON, F32, WS, BIG, None) == -2
assert lib.spec_debug_enable(0) == 1
for code in range(-9, 1):
    assert lib.spec_verify_strerror(code)
assert b"gfx950" in lib.spec_verify_version()
print("host checks ok")
