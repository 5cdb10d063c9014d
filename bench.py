#!/usr/bin/env python3
"""Throughput of the speculative-sampling verify step on one MI355X.

One step = one call of the whole verify path (row sweep, acceptance scan,
replacement/bonus draw with its fp64 fallback for uncertified draws) over
one batch of the headline workload:
B=256 sequences, K=8 drafts, V=128256, bf16 logits, T=0.7.  Inputs are
generated on the host, copied to HBM once, and stay resident; the timed
region is K back-to-back steps between two synchronisations.  The whole
input (1.1 GB) exceeds the 256 MB Infinity Cache, so no step is served from
a previous step's cache.

Warm-up is untimed and lasts at least --warmup steps and at least
--ramp-seconds of them, because a freshly started GPU raises its clocks
over about the first second; the steps it took are reported (`ramp_steps`).

Prints one JSON line.  `value` and `ms_per_step` come from a first timed
pass of K steps with nothing else in the stream.  A second timed pass of K
steps records events between steps (`step_us`: median, p10, p90, first and
last step) and, with each of the sweep's dispatches, events that time every
sweep launch on its own (spec_verify_sweep_timed): `sweep_us` is the sweep
phase (first sweep launch's start to the last one's end, the acceptance
launches between rounds included) and `sweep_launches_us` the sweep launches
alone; those events cost the step some microseconds, so that pass's mean is
reported separately (`ms_per_step_with_events`).  `roofline` describes the
dominant kernel, the row sweep, from its launches' own durations.
`cpu_baseline` times the fp64 oracle on the same batch on all host threads
and on one.

--copy-calibration BYTES first runs three plain device-to-device copies of
that many bytes, so that a rocprofv3 counter pass over the same process
(FETCH_SIZE, WRITE_SIZE) also measures a kernel of known traffic: the ratio
of its known bytes to its counter reading scales the sweep's counters to
bytes.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import functools
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published peak
LLC_BYTES = 256 << 20            # MI355X last-level (Infinity) cache


def input_copies(nbytes: int) -> int:
    """Device copies of a step's input to rotate through: enough that at least
    twice the last-level cache is read between two uses of one copy, so no
    step is served from what the previous use of its input left there."""
    return max(2, -(-2 * LLC_BYTES // max(nbytes, 1)) + 1)
HEADLINE = 2
# The library's sweep rounds (levels [0, 1), [1, 3), [3, K + 1)) unless every
# row's log Z is asked for; used here only to count the bytes a step reads.
ROUND_BEGINS = (0, 1, 3)
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "sweep_headline_counters.md")
# the sweep phase's sources: its kernels, the headers they include and the
# host code that sets their launch shapes (hashed in this order)
SWEEP_SOURCES = [os.path.join(ROOT, "speculative_sampling_verify_spec_amd", "csrc", f)
                 for f in ("k_sweep.hip", "k_rounds.hip", "sv_device.h", "sv_internal.h", "api.cpp")]


def sweep_source_sha256() -> str:
    h = hashlib.sha256()
    for f in SWEEP_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t pairs from the HIP runtime torch already loaded."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0 and self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a.value, b.value))

    def between_ms(self, a: int, b: int) -> float:
        """From the start event of pair a to the end event of pair b."""
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), self.pairs[a][0], self.pairs[b][1]) == 0
        return ms.value

    def elapsed_ms(self, i: int) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), *self.pairs[i]) == 0
        return ms.value

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


def counter_traffic(swept_bytes: int):
    """HBM bytes of the sweep phase per step from the committed rocprofv3
    counter summary, or None when it is missing or was taken on different
    sweep kernels."""
    if not os.path.exists(COUNTER_SUMMARY):
        return None
    text = open(COUNTER_SUMMARY).read()
    src = sweep_source_sha256()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.e+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src:
        return None
    return float(m_bytes.group(1))


def acceptance_summary(n, kb, K: int) -> dict:
    """Acceptance as the pages' monitoring advice asks for it ([D] "Мониторинг в
    производстве": acceptance by position), from one call's counts: the share
    of the sequences that tested position k (k < K_b, no rejection before k)
    that accepted it; the overall rate beta over all tests; the tokens a round
    emits (accepted + 1) as measured, and as the pages' formula predicts for
    i.i.d. acceptance beta and K drafts ([B] "加速比公式：什么时候值得投机？":
    E[N] = (1 - beta^(K+1)) / (1 - beta))."""
    import numpy as np
    n, kb = np.asarray(n), np.asarray(kb)
    tested = np.array([int(np.sum((n >= k) & (kb > k))) for k in range(K)])
    accepted = np.array([int(np.sum(n > k)) for k in range(K)])
    beta = float(accepted.sum() / max(tested.sum(), 1))
    pred = float(K + 1) if beta >= 1.0 else (1.0 - beta ** (K + 1)) / (1.0 - beta)
    return {"per_position": [round(float(a / t), 4) if t else None for a, t in zip(accepted, tested)],
            "tested": tested.tolist(), "beta": round(beta, 4),
            "tokens_per_round": float(np.mean(n + 1)), "tokens_per_round_predicted_iid": round(pred, 4)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Oracle threads: the host's cores, at most 16 (one GPU's share of a
    shared host)."""
    return max(1, min(16, os.cpu_count() or 1))


def cpu_baseline(batch, gpu_tokens, gpu_n, budget_s: float):
    """The fp64 oracle, as it stands, on the timed batch, in the same run:
    whole passes over its sequences on all host threads (numpy releases the
    interpreter lock in its array operations), then on one thread, each for
    about half of budget_s (at least one pass / one sequence).  The all-thread
    rate is `value`.  Also counts sequences whose GPU output differs."""
    import numpy as np
    from oracle import verify_batch
    threads = host_threads()
    # all threads: whole passes over the batch
    passes, mismatched, t0 = 0, 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s / 2 or passes == 0:
        r = verify_batch(batch, workers=threads)
        if passes == 0:
            mismatched = int(np.sum((r.n_accepted != gpu_n) | np.any(r.tokens != gpu_tokens, axis=1)))
        passes += 1
    dt_all = time.perf_counter() - t0
    # one thread: sequence by sequence
    done, t1 = 0, time.perf_counter()
    while time.perf_counter() - t1 < budget_s / 2 or done == 0:
        verify_batch(batch, seqs=[done % batch.B])
        done += 1
    dt_one = time.perf_counter() - t1
    return {"value": passes * batch.B / dt_all, "unit": "verified seq-steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} whole passes over the timed batch of {batch.B} sequences, fp64 numpy, "
                      f"{threads} threads",
            "seconds": round(dt_all, 2),
            "one_thread": {"value": done / dt_one, "sample": f"{done} sequence verifications, one thread",
                           "seconds": round(dt_one, 2)},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample_mismatches_vs_gpu": mismatched, "sample_compared": batch.B}


def rows_per_step(n, kb, K: int, greedy: bool, full: bool):
    """Logit rows one step reads (the sweep only), and the rows the method
    needs: levels 0..n of each sequence (target row k, and draft row k below
    K_b), n its accepted count.  The full sweep reads every row up to K_b; the
    rounds read a round's rows for every sequence that reached it (no
    rejection before its first level)."""
    import numpy as np
    n, kb = np.asarray(n, np.int64), np.asarray(kb, np.int64)
    drafts = 0 if greedy else 1
    needed = int(np.sum((n + 1) + drafts * np.minimum(n + 1, kb)))
    if full:
        return int(np.sum((kb + 1) + drafts * kb)), needed
    bounds = [b for b in ROUND_BEGINS if b <= K] + [K + 1]
    read = 0
    for a, b in zip(bounds[:-1], bounds[1:]):
        reached = n >= a
        t = np.clip(np.minimum(b - 1, kb) - a + 1, 0, None)
        d = np.clip(np.minimum(b, kb) - a, 0, None)
        read += int(np.sum(np.where(reached, t + drafts * d, 0)))
    return read, needed


def dist_us(ms) -> dict:
    """Median, p10, p90, mean, first and last of per-step times (ms in, us out)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "mean": float(np.mean(a)), "first": float(a[0]), "last": float(a[-1]), "n": int(a.size)}


def warm_up(step, steps: int, seconds: float):
    """Untimed warm-up: at least `steps` steps and at least `seconds` of them
    (the clocks of a freshly started GPU rise over the first second or so).
    Returns the steps taken and a trace of their mean time per block."""
    import torch
    done, t0, trace = 0, time.perf_counter(), []
    tb, nb = t0, 0
    while done < steps or time.perf_counter() - t0 < seconds:
        step()
        done += 1
        nb += 1
        if nb == 200:  # bound the queue, and record how the step time settles
            torch.cuda.synchronize()
            now = time.perf_counter()
            trace.append(round((now - tb) / nb * 1e6, 1))
            tb, nb = now, 0
    torch.cuda.synchronize()
    return done, time.perf_counter() - t0, trace


def tree_rows_read(lg, tokens, parents, dtype: str, rounds: bool) -> int:
    """Node rows the library reads for a batch of trees: every row in one
    sweep, or in rounds by depth (the roots; depths 1-2 under an accepted
    depth-1 ancestor; deeper nodes under an accepted depth-3 ancestor), a node
    being accepted when its token is its parent's first arg-max and its
    parent is accepted (host arithmetic on the batch, for the byte count)."""
    import numpy as np
    B, N = tokens.shape
    if not rounds or N == 1:
        return B * N
    rows = (lg.astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else lg
    amax = np.stack([np.argmax(rows[b], axis=1) for b in range(B)])
    total = 0
    for b in range(B):
        par = parents[b]
        depth = np.zeros(N, int)
        acc = np.zeros(N, bool)
        anc = [[0] for _ in range(N)]  # ancestors from the root down, the node last
        acc[0] = True
        for v in range(1, N):
            pv = int(par[v])
            if 0 <= pv < v:
                depth[v] = depth[pv] + 1
                acc[v] = acc[pv] and int(tokens[b, v]) == int(amax[b, pv])
                anc[v] = anc[pv] + [v]
            else:
                anc[v] = [v]
                depth[v] = 0
        total += 1
        for v in range(1, N):
            d, a = depth[v], anc[v]
            valid = a[0] == 0
            if valid and 1 <= d < 3 and acc[a[1]]:
                total += 1
            elif valid and d >= 3 and acc[a[3]]:
                total += 1
    return total


def tree_bench(args):
    """Greedy token-tree verification: B trees of N nodes over V=128256 bf16
    logits (in rounds by depth: only rows below accepted nodes are read)."""
    import numpy as np
    import torch

    import speculative_sampling_verify_spec_amd as sv
    import workloads
    B, N, V = 128, 32, 128256
    log(f"generating {B} trees of {N} nodes, V={V} bf16")
    tb = workloads.make_tree_batch(B, N, V, "bf16", workers=workloads.default_workers())
    lg = torch.from_numpy(tb.logits.view(np.int16)).cuda().view(torch.bfloat16)
    ncopy = input_copies(lg.numel() * 2)
    lgs = [lg] + [lg.clone() for _ in range(ncopy - 1)]  # used in turn
    tok_in = torch.from_numpy(tb.tokens).cuda()
    par = torch.from_numpy(tb.parents).cuda()
    ws = torch.empty(int(sv.load().spec_verify_tree_workspace_size(B, N, V, sv.SPECV_BF16)), dtype=torch.uint8,
                     device="cuda")
    turn = [0]

    def warm():
        sv.verify_tree_greedy(lgs[turn[0] % ncopy], tok_in, par, workspace=ws)
        turn[0] += 1
    ramp_steps, _, _ = warm_up(warm, args.warmup, args.ramp_seconds)
    t0 = time.perf_counter()
    for i in range(args.steps):
        out = sv.verify_tree_greedy(lgs[i % ncopy], tok_in, par, workspace=ws)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    n = out[2].cpu().numpy()
    nbytes = B * N * V * 2
    rounds = nbytes >= sv.rounds_min_bytes()
    rows_read = tree_rows_read(tb.logits, tb.tokens, tb.parents, "bf16", rounds)
    read = rows_read * V * 2
    line = {"metric": "verified trees/s + HBM GB/s (% peak), greedy token trees", "value": B / step_s,
            "unit": "verified trees/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ramp_steps": ramp_steps,
            "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"tree-bf16: {B} trees of {N} nodes (chains branching with probability 1/2), "
                                   f"V={V} bf16, greedy", "B": B, "N": N, "V": V},
            "rounds": bool(rounds),
            # the node rows the library reads (in rounds by depth, only those below accepted nodes)
            "hbm_gbps": read / step_s / 1e9, "hbm_frac_of_peak": read / step_s / 1e9 / PEAK_HBM_GBS,
            # every node row once, per step time: above peak when rounds skip rows
            "hbm_gbps_all_rows_model": nbytes / step_s / 1e9,
            "bytes_per_step": {"read": read, "rows_read": rows_read, "all_rows": nbytes, "rows_all": B * N},
            "mean_accepted": float(np.mean(n)), "input_copies": ncopy, "roofline": None,
            "cpu_baseline": None}
    if not args.no_cpu_baseline:
        from oracle import tree
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds or done == 0:
            b = done % B
            tree.verify_tree_greedy_sequence(tb.logits[b], tb.tokens[b], tb.parents[b], "bf16")
            done += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": done / dt, "unit": "verified trees/s", "cores": 1, "kind": "oracle",
                                "sample": f"{done} tree verifications of the timed batch, numpy, one thread",
                                "seconds": round(dt, 2)}
    print(json.dumps(line), flush=True)


def ngram_bench(args):
    """Prompt-lookup proposals for B histories (every history token read once)."""
    import numpy as np
    import torch

    import speculative_sampling_verify_spec_amd as sv
    import workloads
    B, L, vocab, n_min, n_max, hits, K = 1024, 16384, 32000, 1, 4, 1, 5
    log(f"generating {B} histories of up to {L} tokens")
    hist, lens = workloads.make_histories(B, L, vocab, workers=workloads.default_workers())
    h, ln = torch.from_numpy(hist).cuda(), torch.from_numpy(lens).cuda()
    ncopy = input_copies(h.numel() * 4)
    hs = [h] + [h.clone() for _ in range(ncopy - 1)]  # used in turn
    turn = [0]

    def warm():
        sv.ngram_propose(hs[turn[0] % ncopy], ln, n_min, n_max, hits, K)
        turn[0] += 1
    ramp_steps, _, _ = warm_up(warm, args.warmup, args.ramp_seconds)
    t0 = time.perf_counter()
    for i in range(args.steps):
        out = sv.ngram_propose(hs[i % ncopy], ln, n_min, n_max, hits, K)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    nbytes = int(np.sum(lens)) * 4
    cnt = out[1].cpu().numpy()
    line = {"metric": "proposals/s + HBM GB/s (% peak), n-gram prompt lookup", "value": B / step_s,
            "unit": "proposals/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ramp_steps": ramp_steps,
            "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "int32", "data": "synthetic",
            "config": {"workload": f"ngram: {B} histories, lengths uniform in [{L // 2}, {L}], vocab {vocab}, "
                                   f"copies of earlier spans with probability 1/2; n = {n_min}..{n_max}, "
                                   f"min hits {hits}, K = {K}", "B": B, "L_max": L},
            "hbm_gbps_algorithmic": nbytes / step_s / 1e9, "hbm_frac_of_peak": nbytes / step_s / 1e9 / PEAK_HBM_GBS,
            "bytes_per_step": nbytes, "proposal_rate": float(np.mean(cnt > 0)), "mean_draft": float(np.mean(cnt)),
            "input_copies": ncopy,
            "roofline": None, "cpu_baseline": None}
    if not args.no_cpu_baseline:
        from oracle import ngram
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds or done == 0:
            b = done % B
            ngram.propose_sequence(hist[b, : lens[b]], n_min, n_max, hits, K)
            done += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": done / dt, "unit": "proposals/s", "cores": 1, "kind": "oracle",
                                "sample": f"{done} histories of the timed batch, numpy, one thread",
                                "seconds": round(dt, 2)}
    print(json.dumps(line), flush=True)


def ngram_map_bench(args):
    """The n-gram map on the n-gram workload's histories: one table per history,
    built once, then one update per step that adds the tokens a step appends to
    every history (K + 1: every draft accepted, plus the bonus token) and
    proposes.  The scan (spec_ngram_propose) is timed on the same lengths."""
    import numpy as np
    import torch

    import speculative_sampling_verify_spec_amd as sv
    import workloads
    lib = sv.load()
    B, L, vocab, n_min, n_max, hits, K = 1024, 16384, 32000, 1, 4, 1, 5
    add = K + 1
    cap = 1 << (2 * (n_max - n_min + 1) * L - 1).bit_length()
    log(f"generating {B} histories of up to {L} tokens; tables of {cap} slots")
    hist, lens = workloads.make_histories(B, L, vocab, workers=workloads.default_workers())
    nsteps = args.warmup + args.steps
    start = lens - add * nsteps
    if start.min() < 1:
        print("--warmup + --steps too large for these histories", file=sys.stderr)
        sys.exit(2)
    steps_len = np.stack([start + add * i for i in range(nsteps + 1)]).astype(np.int32)  # [step][B]
    h = torch.from_numpy(hist).cuda()
    lens_dev = torch.from_numpy(steps_len).cuda()
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")
    nbytes = sv.ngram_map_bytes(B, cap)
    tables = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    spare = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    draft = torch.empty((B, K), dtype=torch.int32, device="cuda")
    count = torch.empty(B, dtype=torch.int32, device="cuda")
    status = torch.empty(B, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    fn = lib.spec_ngram_map_update

    def upd(tab, old_ptr, new_ptr):
        return functools.partial(fn, P(tab), cap, P(h), old_ptr, new_ptr, B, L, n_min, n_max, hits, K, P(draft),
                                 P(count), P(status), st)
    row = lambda i: P(lens_dev) + 4 * B * i
    build_spare = upd(spare, P(zeros), row(0))
    ramp_steps, _, _ = warm_up(lambda: build_spare(), 1, args.ramp_seconds)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    assert upd(tables, P(zeros), row(0))() == 0
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0
    calls = [upd(tables, row(i), row(i + 1)) for i in range(nsteps)]
    for c in calls[:args.warmup]:
        c()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for c in calls[args.warmup:]:
        c()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    map_draft, map_count, map_status = draft.cpu().numpy(), count.cpu().numpy(), status.cpu().numpy()
    # the scan on the final lengths, the same number of calls
    final = lens_dev[nsteps]
    sd = torch.empty((B, K), dtype=torch.int32, device="cuda")
    sc = torch.empty(B, dtype=torch.int32, device="cuda")
    scan = functools.partial(lib.spec_ngram_propose, P(h), P(final), B, L, n_min, n_max, hits, K, P(sd), P(sc), st)
    for _ in range(args.warmup):
        scan()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        scan()
    torch.cuda.synchronize()
    scan_s = (time.perf_counter() - t0) / args.steps
    mism = int(np.sum(np.any(map_draft != sd.cpu().numpy(), axis=1) | (map_count != sc.cpu().numpy())))
    line = {"metric": "proposals/s, n-gram map update + lookup", "value": B / step_s, "unit": "proposals/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ramp_steps": ramp_steps,
            "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "int32", "data": "synthetic",
            "config": {"workload": f"ngram map: {B} histories, lengths uniform in [{L // 2}, {L}] less "
                                   f"{add * nsteps} tokens at the build, {add} tokens added per history per "
                                   f"step; vocab {vocab}, n = {n_min}..{n_max}, min hits {hits}, K = {K}",
                       "B": B, "L_max": L, "capacity": cap, "table_bytes": nbytes},
            "build_ms": build_s * 1e3, "scan_ms_per_step_same_lengths": scan_s * 1e3,
            "map_vs_scan_mismatches": mism, "tables_full": int(np.count_nonzero(map_status)),
            "proposal_rate": float(np.mean(map_count > 0)), "mean_draft": float(np.mean(map_count)),
            "roofline": None, "cpu_baseline": None}
    if not args.no_cpu_baseline:
        from oracle import ngram
        fl = steps_len[nsteps]
        done, bad, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds or done == 0:
            b = done % B
            d, c = ngram.propose_sequence(hist[b, : fl[b]], n_min, n_max, hits, K)
            bad += int(c != map_count[b] or np.any(d != map_draft[b]))
            done += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": done / dt, "unit": "proposals/s", "cores": 1, "kind": "oracle",
                                "sample": f"{done} histories at the final lengths, numpy scan, one thread",
                                "seconds": round(dt, 2), "sample_mismatches_vs_map": bad}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--ramp-seconds", type=float, default=2.0,
                    help="untimed warm-up lasts at least this long, whatever --warmup says (clock ramp)")
    ap.add_argument("--workload", type=int, default=HEADLINE, choices=range(5))
    ap.add_argument("--seqs", type=int, default=0, metavar="N",
                    help="verify sequences 0..N-1 of the workload's seeded recipe instead of its B (a smaller "
                         "or larger batch of the same shape)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--tree", action="store_true",
                    help="greedy token-tree verification: 128 trees of 32 nodes, V=128256 bf16")
    ap.add_argument("--ngram", action="store_true",
                    help="prompt-lookup proposer: 1024 histories of up to 16384 tokens, n = 1..4, K = 5")
    ap.add_argument("--ngram-map", action="store_true",
                    help="n-gram map: the --ngram histories in hash tables, built once, then updated with 6 "
                         "tokens per history per step")
    ap.add_argument("--full", action="store_true",
                    help="ask for every row's log Z, which sweeps every row at once instead of in rounds")
    ap.add_argument("--ragged", action="store_true",
                    help="per-sequence draft counts K_b uniform on [1, K] (spec_verify_ragged with "
                         "per-position counters); bytes count the rows actually read")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the verify step is data-parallel "
              "over sequences and a multi-GPU run would shard B across processes", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_sampling_verify_spec_amd as sv
    import workloads

    sv.load()
    if args.tree:
        tree_bench(args)
        return
    if args.ngram:
        ngram_bench(args)
        return
    if args.ngram_map:
        ngram_map_bench(args)
        return
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 device copies of {args.copy_calibration} bytes")
        del src, dst
    wl = workloads.WORKLOADS[args.workload]
    if args.seqs < 0:
        print("--seqs must be positive", file=sys.stderr)
        sys.exit(2)
    seqs = range(args.seqs) if args.seqs else None
    log(f"generating {wl.name}: {wl.describe()}" + (f", sequences 0..{args.seqs - 1}" if args.seqs else ""))
    t0 = time.perf_counter()
    batch = workloads.make_batch(args.workload, seqs=seqs, workers=workloads.default_workers())
    log(f"generated in {time.perf_counter() - t0:.1f}s; copying to HBM")
    lp, lq, x, ua, ur = workloads.to_device(batch)
    B, K, V, T = batch.B, batch.K, batch.V, batch.T
    greedy = T == 0.0
    elt = 2 if batch.dtype == "bf16" else 4
    dt_code = sv.SPECV_BF16 if batch.dtype == "bf16" else sv.SPECV_F32
    ws = torch.empty(sv.workspace_size(B, K, V, dt_code, T), dtype=torch.uint8, device="cuda")
    tokens = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    n_acc = torch.empty((B,), dtype=torch.int32, device="cuda")
    flags = torch.empty((B,), dtype=torch.int32, device="cuda")
    logz = torch.empty((B, 2 * K + 1), dtype=torch.float32, device="cuda") if args.full else None
    nev = len(ROUND_BEGINS)  # sweep launches per call, at most
    ev = HipEvents(args.steps * nev)
    nsweeps = []

    kb_host = workloads.ragged_draft_counts(B, K) if args.ragged else None
    if args.ragged:
        batch = dataclasses.replace(batch, num_drafts=kb_host)  # the oracle baseline verifies the same counts
    kb = torch.from_numpy(kb_host).cuda() if args.ragged else None
    stats = torch.zeros(2 * K, dtype=torch.int64, device="cuda")

    # the logits in several device copies, used in turn (the draft tokens and
    # uniforms, a few KB, are shared)
    ncopy = input_copies(lp.numel() * lp.element_size() + (0 if lq is None else lq.numel() * lq.element_size()))
    copies = [(lp, lq)] + [(lp.clone(), None if lq is None else lq.clone()) for _ in range(ncopy - 1)]
    turn = [0]

    # the same calls with their arguments marshalled once per input copy, so
    # that the timed loop measures the library rather than Python
    if args.ragged:
        bound = [sv.bind_spec_verify_ragged(cp, cq, x, kb, ua, ur, T, tokens, n_acc, ws, position_stats=stats,
                                            out_logz=logz) for cp, cq in copies]
    else:
        bound = [sv.bind_spec_verify(cp, cq, x, ua, ur, T, tokens, n_acc, ws, out_flags=flags, out_logz=logz,
                                     extended=True) for cp, cq in copies]

    def step(e=None):
        cp, cq = copies[turn[0] % ncopy]
        call = bound[turn[0] % ncopy]
        turn[0] += 1
        if e is None:
            rc = call()
        else:  # step e of the events pass: a pair of events per sweep launch
            pairs = ev.pairs[e * nev:(e + 1) * nev]
            rc, ns = sv.spec_verify_sweep_timed(cp, cq, x, ua, ur, T, tokens, n_acc, ws,
                                                [a for a, _ in pairs], [b for _, b in pairs],
                                                out_logz=logz, out_flags=flags)
            nsweeps.append(ns)
        if rc != 0:
            raise RuntimeError(sv.strerror(rc))

    ramp_steps, ramp_s, ramp_trace = warm_up(step, args.warmup, args.ramp_seconds)
    log(f"warm after {ramp_steps} steps ({ramp_s:.2f}s; us per step by blocks of 200: {ramp_trace[:12]}"
        f"{' ...' if len(ramp_trace) > 12 else ''}); timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # a second pass of K steps: events between steps (per-step times) and,
    # outside ragged mode, events recorded with the sweep's dispatches
    log(f"timing {args.steps} steps with events")
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    bounds[0].record()
    for i in range(args.steps):
        step(None if args.ragged else i)
        bounds[i + 1].record()
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t0
    step_ms = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)]
    # per step: the sweep phase, and the sweep launches' own durations summed
    sweep_ms = None if args.ragged else [ev.between_ms(i * nev, i * nev + nsweeps[i] - 1) for i in range(args.steps)]
    launches_ms = None if args.ragged else [sum(ev.elapsed_ms(i * nev + r) for r in range(nsweeps[i]))
                                            for i in range(args.steps)]
    ev.close()

    n_host = n_acc.cpu().numpy()
    tok_host = tokens.cpu().numpy()
    kbs = kb_host if args.ragged else np.full(B, K)
    rows_all = int(np.sum(kbs + 1)) if greedy else int(np.sum(2 * kbs + 1))
    # one sweep of every row when asked for, or when the call's B (K + 1) +
    # B K logit rows (B (K + 1) greedy) are below the library's rounds
    # threshold (its default, 256 MiB)
    full = args.full or (B * (K + 1 if greedy else 2 * K + 1) * V * elt < 256 * 2 ** 20)
    rows_read, rows_needed = rows_per_step(n_host, kbs, K, greedy, full)
    swept, needed, swept_all = (r * V * elt for r in (rows_read, rows_needed, rows_all))
    reread = 0 if greedy else int(np.sum(np.where(n_host < kbs, 2, 1))) * V * elt
    step_s = wall / args.steps
    line = {
        "metric": f"verified seq-steps/s + HBM GB/s (% peak), B={B} K={K} V={V} {batch.dtype}",
        "value": B / step_s,
        "unit": "verified seq-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "ms_per_step_with_events": wall_ev / args.steps * 1e3,
        "ramp_steps": ramp_steps, "ramp_seconds": round(ramp_s, 3),
        "step_us": dist_us(step_ms),
        "sweep_us": None if sweep_ms is None else dist_us(sweep_ms),
        "sweep_launches_us": None if launches_ms is None else dist_us(launches_ms),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{wl.name}: verify {batch.wl.describe()}, logits {batch.dtype}"
                               + (f" (the first {B} sequences of the {wl.B})" if args.seqs else "")
                               + (", per-sequence draft counts uniform on [1, K]" if args.ragged else "")
                               + (", every row's log Z (one sweep of every row)" if args.full else ""),
                   "B": B, "K": K, "V": V, "logits": batch.dtype, "T": T, "parallelism": "none (one GPU)"},
        # bytes the step reads from HBM (rows swept + decisive rows reread)
        "hbm_gbps": (swept + reread) / step_s / 1e9,
        "hbm_frac_of_peak": (swept + reread) / step_s / 1e9 / PEAK_HBM_GBS,
        # every logit once + the reread (the byte count the headline metric
        # names), per step time: above peak when rows past a rejection are skipped
        "hbm_gbps_all_rows_model": (swept_all + reread) / step_s / 1e9,
        "bytes_per_step": {"swept": swept, "decisive_reread": reread, "rows_swept": rows_read,
                           "needed": needed, "rows_needed": rows_needed, "all_rows": swept_all,
                           "rows_all": rows_all},
        "mean_accepted": float(np.mean(n_host)),
        "acceptance": acceptance_summary(n_host, kb_host if args.ragged else np.full(B, K), K),
        "input_copies": ncopy,
        "fp64_draw_fraction": None if (greedy or args.ragged) else float(np.mean((flags.cpu().numpy() & sv.FLAG_FP64) != 0)),
        "roofline": None,
        "cpu_baseline": None,
    }
    if args.ragged:
        line["position_stats"] = stats.cpu().numpy().tolist()
    else:
        nr = nsweeps[0]
        assert all(n == nr for n in nsweeps), nsweeps
        assert nr == (1 if full else len([b for b in ROUND_BEGINS if b <= K])), nr
        launches_s = float(np.mean(launches_ms)) / 1e3  # the sweep launches of one step, summed
        phase_s = float(np.mean(sweep_ms)) / 1e3
        achieved = swept / launches_s / 1e9
        kname = "k_sweep_lse" if not greedy else "k_sweep_argmax"
        line["roofline"] = {"bound": "hbm",
                            "kernel": f"row sweep: {kname}, " + ("one launch per step" if nr == 1 else
                                      f"{nr} round launches per step, each timed with HIP events recorded "
                                      "with its own dispatch"),
                            "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": achieved / PEAK_HBM_GBS,
                            # the committed counters cover the headline's log-sum-exp sweep
                            "traffic": None if (greedy or args.full or args.seqs or args.workload != HEADLINE)
                            else counter_traffic(swept),
                            "launch_us": launches_s / nr * 1e6, "launches_timed": args.steps * nr,
                            "sweep_launches_per_step": nr,
                            "algorithmic_bytes_per_launch": swept / nr,
                            "algorithmic_bytes": "the logit rows the sweep reads (rows of the positions each "
                                                 "sequence reached), V * element size each; per launch, the "
                                                 "step's rows over its launches",
                            # the sweep phase: first sweep launch's start to the last one's end, with the
                            # acceptance launches between the rounds
                            "sweep_phase_us": phase_s * 1e6,
                            "sweep_phase_frac": swept / phase_s / 1e9 / PEAK_HBM_GBS}
    if not args.no_cpu_baseline:
        log(f"timing the fp64 oracle on a sample (~{args.cpu_seconds:.0f}s)")
        line["cpu_baseline"] = cpu_baseline(batch, tok_host, n_host, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
