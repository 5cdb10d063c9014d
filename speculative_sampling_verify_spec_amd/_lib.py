"""ctypes binding of libspecverify (argument marshalling only).

Every step of the verify pass runs in the library's HIP kernels; this module
checks shapes and dtypes, allocates outputs and the workspace with torch, and
passes raw device pointers plus torch's current HIP stream.  There is no CPU
fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")

SPECV_F32, SPECV_BF16 = 0, 1
SPECV_MAX_K = 32
SPECV_MAX_TREE = 64
SPECV_MAX_NGRAM = 16
FLAG_FP64, FLAG_ZW_ZERO, FLAG_BAD_DRAFT = 1, 2, 4

ERRORS = {0: "SPECV_OK", -1: "SPECV_E_NULL", -2: "SPECV_E_SHAPE", -3: "SPECV_E_DTYPE", -4: "SPECV_E_TEMP",
          -5: "SPECV_E_WORKSPACE", -6: "SPECV_E_ALIGN", -7: "SPECV_E_HIP", -8: "SPECV_E_SCRATCH"}
NOALLOC_SCRATCH = 32 << 20
# device-side validation counters (spec_debug_counters), in this order
DEBUG_COUNTERS = ("calls", "bad_draft_ids", "bad_u_accept", "bad_u_resample", "nan_logits", "inf_logits",
                  "rows_no_finite")

# every symbol include/specverify.h declares
EXPORTS = ("spec_verify_workspace_size", "spec_verify", "spec_verify_noalloc", "spec_verify_ex",
           "spec_verify_sweep_timed",
           "spec_verify_ragged",
           "spec_verify_ragged_ex", "spec_verify_tree_workspace_size", "spec_verify_tree_greedy", "spec_tree_mask", "spec_ngram_propose",
           "spec_ngram_map_bytes", "spec_ngram_map_update", "spec_rounds_min_bytes", "spec_short_max_seqs",
           "spec_debug_enable", "spec_debug_counters", "spec_debug_reset",
           "spec_verify_strerror", "spec_verify_version")

_lib: Optional[ctypes.CDLL] = None


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the built library (raises FileNotFoundError if it was never built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # torch first: its bundled HIP runtime carries the same soname, so the
    # library binds to the one runtime instance torch's streams belong to
    import torch  # noqa: F401
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} is missing: build it with `python -m speculative_sampling_verify_spec_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.spec_verify_workspace_size.argtypes = [i32, i32, i32, i32, f32]
    lib.spec_verify_workspace_size.restype = sz
    common = [vp, vp, vp, vp, vp, f32, i32, i32, i32, vp, vp, i32, vp, sz, vp]
    lib.spec_verify.argtypes = common
    lib.spec_verify.restype = i32
    lib.spec_verify_noalloc.argtypes = common[:12] + [vp]
    lib.spec_verify_noalloc.restype = i32
    lib.spec_verify_ex.argtypes = common + [vp, vp, vp, vp]
    lib.spec_verify_ex.restype = i32
    lib.spec_verify_sweep_timed.argtypes = common + [vp, vp, vp, vp, i32, vp]
    lib.spec_verify_sweep_timed.restype = i32
    ragged = [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.spec_verify_ragged.argtypes = ragged
    lib.spec_verify_ragged.restype = i32
    lib.spec_verify_ragged_ex.argtypes = ragged + [vp, vp]
    lib.spec_verify_ragged_ex.restype = i32
    lib.spec_verify_tree_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.spec_verify_tree_workspace_size.restype = sz
    lib.spec_verify_tree_greedy.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.spec_verify_tree_greedy.restype = i32
    lib.spec_tree_mask.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.spec_tree_mask.restype = i32
    lib.spec_ngram_propose.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.spec_ngram_propose.restype = i32
    lib.spec_rounds_min_bytes.argtypes = [ctypes.c_double]
    lib.spec_rounds_min_bytes.restype = ctypes.c_double
    lib.spec_short_max_seqs.argtypes = [ctypes.c_int]
    lib.spec_short_max_seqs.restype = ctypes.c_int
    lib.spec_ngram_map_bytes.argtypes = [i32, i32]
    lib.spec_ngram_map_bytes.restype = sz
    lib.spec_ngram_map_update.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.spec_ngram_map_update.restype = i32
    lib.spec_debug_enable.argtypes = [i32]
    lib.spec_debug_enable.restype = i32
    lib.spec_debug_counters.argtypes = [vp, i32]
    lib.spec_debug_counters.restype = i32
    lib.spec_debug_reset.argtypes = []
    lib.spec_debug_reset.restype = i32
    lib.spec_verify_strerror.argtypes = [i32]
    lib.spec_verify_strerror.restype = ctypes.c_char_p
    lib.spec_verify_version.argtypes = []
    lib.spec_verify_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().spec_verify_strerror(code).decode()


def version() -> str:
    return load().spec_verify_version().decode()


def debug_enable(on: bool) -> bool:
    """Turn device-side input validation on or off for later verify calls;
    returns the previous setting."""
    return bool(load().spec_debug_enable(1 if on else 0))


def debug_counters() -> dict:
    """The current device's validation counters (synchronises the device)."""
    buf = (ctypes.c_ulonglong * len(DEBUG_COUNTERS))()
    rc = int(load().spec_debug_counters(ctypes.cast(buf, ctypes.c_void_p), len(DEBUG_COUNTERS)))
    if rc != 0:
        raise SpecVerifyError(rc, strerror(rc))
    return dict(zip(DEBUG_COUNTERS, (int(v) for v in buf)))


def debug_reset() -> None:
    """Zero the current device's validation counters (synchronises the device)."""
    rc = int(load().spec_debug_reset())
    if rc != 0:
        raise SpecVerifyError(rc, strerror(rc))


def workspace_size(B: int, K: int, V: int, dtype: int, T: float) -> int:
    return int(load().spec_verify_workspace_size(B, K, V, dtype, T))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SPECV_BF16
    if t.dtype == torch.float32:
        return SPECV_F32
    raise TypeError(f"logits must be torch.bfloat16 or torch.float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _spec_verify_call(logits_p, logits_q, draft_tokens, u_accept, u_resample, T, out_tokens, out_n_accepted,
                      workspace, out_logz, out_flags, events, stream, extended):
    """The library function and its argument list for one spec_verify(_ex) call."""
    lib = load()
    B, K1, V = logits_p.shape
    K = K1 - 1
    dt = _dtype_code(logits_p)
    import torch
    st = stream if stream is not None else torch.cuda.current_stream(logits_p.device).cuda_stream
    args = [_ptr(logits_p), _ptr(logits_q), _ptr(draft_tokens), _ptr(u_accept), _ptr(u_resample),
            float(T), B, K, V, _ptr(out_tokens), _ptr(out_n_accepted), dt,
            _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(), st]
    if not extended and out_logz is None and out_flags is None and events is None:
        return lib.spec_verify, args
    e0, e1 = events if events is not None else (None, None)
    return lib.spec_verify_ex, args + [_ptr(out_logz), _ptr(out_flags), e0, e1]


def spec_verify(logits_p, logits_q, draft_tokens, u_accept, u_resample, T: float,
                out_tokens=None, out_n_accepted=None, workspace=None, *,
                out_logz=None, out_flags=None, events=None, stream=None, extended: bool = False) -> int:
    """Raw call with caller-provided device tensors; returns the library's status code."""
    fn, args = _spec_verify_call(logits_p, logits_q, draft_tokens, u_accept, u_resample, T, out_tokens,
                                 out_n_accepted, workspace, out_logz, out_flags, events, stream, extended)
    return int(fn(*args))


def _bound(fn, args):
    """fn with its arguments converted to ctypes values once."""
    conv = [t(a) if a is not None else None for t, a in zip(fn.argtypes, args)]
    return functools.partial(fn, *conv)


def bind_spec_verify(logits_p, logits_q, draft_tokens, u_accept, u_resample, T: float,
                     out_tokens=None, out_n_accepted=None, workspace=None, *,
                     out_logz=None, out_flags=None, stream=None, extended: bool = False):
    """spec_verify's arguments marshalled once: returns a function of no
    arguments that enqueues the same call again and returns its status code,
    for loops over resident buffers (the tensors must stay alive and in
    place)."""
    return _bound(*_spec_verify_call(logits_p, logits_q, draft_tokens, u_accept, u_resample, T, out_tokens,
                                     out_n_accepted, workspace, out_logz, out_flags, None, stream, extended))


def spec_verify_sweep_timed(logits_p, logits_q, draft_tokens, u_accept, u_resample, T: float, out_tokens,
                            out_n_accepted, workspace, ev_begin, ev_end, out_logz=None, out_flags=None,
                            stream=None):
    """spec_verify_sweep_timed on torch device tensors: ev_begin, ev_end are
    sequences of hipEvent_t handles (ints), recorded with each sweep launch in
    turn.  Returns (return code, number of sweep launches)."""
    n = len(ev_begin)
    if len(ev_end) != n:
        raise ValueError("ev_begin and ev_end need the same length")
    beg = (ctypes.c_void_p * max(n, 1))(*ev_begin)
    end = (ctypes.c_void_p * max(n, 1))(*ev_end)
    ns = ctypes.c_int(0)
    _, args = _spec_verify_call(logits_p, logits_q, draft_tokens, u_accept, u_resample, T, out_tokens,
                                out_n_accepted, workspace, out_logz, out_flags, None, stream, True)
    args = args[:-2] + [ctypes.cast(beg, ctypes.c_void_p), ctypes.cast(end, ctypes.c_void_p), n, ctypes.byref(ns)]
    rc = int(load().spec_verify_sweep_timed(*args))
    return rc, int(ns.value)


def spec_verify_noalloc(logits_p, logits_q, draft_tokens, u_accept, u_resample, T: float, out_tokens,
                        out_n_accepted, *, stream=None) -> int:
    """Raw call of spec_verify_noalloc (no workspace: the library's static
    scratch); returns the library's status code."""
    lib = load()
    B, K1, V = logits_p.shape
    import torch
    st = stream if stream is not None else torch.cuda.current_stream(logits_p.device).cuda_stream
    return int(lib.spec_verify_noalloc(_ptr(logits_p), _ptr(logits_q), _ptr(draft_tokens), _ptr(u_accept),
                                       _ptr(u_resample), float(T), B, K1 - 1, V, _ptr(out_tokens),
                                       _ptr(out_n_accepted), _dtype_code(logits_p), st))


def spec_verify_ragged(logits_p, logits_q, draft_tokens, num_drafts, u_accept, u_resample, T: float,
                       out_tokens=None, out_n_accepted=None, workspace=None, *, position_stats=None,
                       out_logz=None, out_flags=None, stream=None) -> int:
    """Raw call of spec_verify_ragged (spec_verify_ragged_ex when log Z or
    flags are asked for); returns the library's status code."""
    fn, args = _spec_verify_ragged_call(logits_p, logits_q, draft_tokens, num_drafts, u_accept, u_resample, T,
                                        out_tokens, out_n_accepted, workspace, position_stats, out_logz, out_flags,
                                        stream)
    return int(fn(*args))


def bind_spec_verify_ragged(logits_p, logits_q, draft_tokens, num_drafts, u_accept, u_resample, T: float,
                            out_tokens=None, out_n_accepted=None, workspace=None, *, position_stats=None,
                            out_logz=None, out_flags=None, stream=None):
    """spec_verify_ragged's arguments marshalled once (see bind_spec_verify)."""
    return _bound(*_spec_verify_ragged_call(logits_p, logits_q, draft_tokens, num_drafts, u_accept, u_resample, T,
                                            out_tokens, out_n_accepted, workspace, position_stats, out_logz,
                                            out_flags, stream))


def _spec_verify_ragged_call(logits_p, logits_q, draft_tokens, num_drafts, u_accept, u_resample, T, out_tokens,
                             out_n_accepted, workspace, position_stats, out_logz, out_flags, stream):
    """The library function and its argument list for one spec_verify_ragged(_ex) call."""
    lib = load()
    B, K1, V = logits_p.shape
    import torch
    st = stream if stream is not None else torch.cuda.current_stream(logits_p.device).cuda_stream
    args = [_ptr(logits_p), _ptr(logits_q), _ptr(draft_tokens), _ptr(num_drafts), _ptr(u_accept),
            _ptr(u_resample), float(T), B, K1 - 1, V, _ptr(out_tokens), _ptr(out_n_accepted),
            _ptr(position_stats), _dtype_code(logits_p), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(), st]
    if out_logz is None and out_flags is None:
        return lib.spec_verify_ragged, args
    return lib.spec_verify_ragged_ex, args + [_ptr(out_logz), _ptr(out_flags)]


def verify(logits_p, logits_q, draft_tokens, u_accept, u_resample, T: float, *,
           return_logz: bool = False, return_flags: bool = False, workspace=None, events=None,
           num_drafts=None, position_stats=None):
    """One verify step on torch device tensors.

    logits_p [B,K+1,V] and logits_q [B,K,V] (bf16 or fp32, contiguous, same
    device), draft_tokens [B,K] int32, u_accept [B,K] and u_resample [B]
    float32; logits_q / u_accept / u_resample may be None when T == 0.
    Returns (tokens [B,K+1] int32, n_accepted [B] int32) plus log Z
    [B,2K+1] float32 and flags [B] int32 when asked.  Runs on torch's current
    stream; nothing synchronises.

    num_drafts [B] int32 (device) gives every sequence its own draft count
    (spec_verify_ragged); position_stats [2K] int64 (device, zeroed by the
    caller) then receives the per-position tested / accepted counts.  With
    num_drafts, log Z rows a sequence does not use are NaN; events are not
    available."""
    import torch
    dev = logits_p.device
    if dev.type != "cuda":
        raise ValueError("logits_p must be a device tensor")
    if logits_p.dim() != 3:
        raise ValueError("logits_p must be [B, K+1, V]")
    B, K1, V = logits_p.shape
    K = K1 - 1
    greedy = float(T) == 0.0
    tensors = [logits_p, draft_tokens] + ([] if greedy else [logits_q, u_accept, u_resample])
    for t in tensors:
        if t.device != dev or not t.is_contiguous():
            raise ValueError("all inputs must be contiguous tensors on the same device")
    if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, K):
        raise ValueError("draft_tokens must be int32 [B, K]")
    if not greedy:
        if logits_q.dtype != logits_p.dtype or tuple(logits_q.shape) != (B, K, V):
            raise ValueError("logits_q must match logits_p's dtype and be [B, K, V]")
        if u_accept.dtype != torch.float32 or tuple(u_accept.shape) != (B, K):
            raise ValueError("u_accept must be float32 [B, K]")
        if u_resample.dtype != torch.float32 or tuple(u_resample.shape) != (B,):
            raise ValueError("u_resample must be float32 [B]")
    else:
        logits_q = u_accept = u_resample = None
    if num_drafts is not None:
        if num_drafts.device != dev or num_drafts.dtype != torch.int32 or tuple(num_drafts.shape) != (B,):
            raise ValueError("num_drafts must be an int32 [B] tensor on the logits' device")
        if events is not None:
            raise ValueError("num_drafts does not combine with events")
    if position_stats is not None:
        if num_drafts is None:
            raise ValueError("position_stats needs num_drafts")
        if position_stats.device != dev or position_stats.dtype != torch.int64 or \
                tuple(position_stats.shape) != (2 * K,) or not position_stats.is_contiguous():
            raise ValueError("position_stats must be a contiguous int64 [2K] tensor on the logits' device")
    dt = _dtype_code(logits_p)
    need = workspace_size(B, K, V, dt, float(T))
    if need == 0:
        raise SpecVerifyError(-2, "invalid shape, dtype or temperature")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
    logz = None
    if return_logz:  # rows a call does not write stay NaN
        logz = torch.full((B, 2 * K + 1), float("nan"), dtype=torch.float32, device=dev)
    flags = torch.empty((B,), dtype=torch.int32, device=dev) if return_flags else None
    if num_drafts is not None:
        rc = spec_verify_ragged(logits_p, logits_q, draft_tokens, num_drafts, u_accept, u_resample, T, tokens,
                                n_acc, workspace, position_stats=position_stats, out_logz=logz, out_flags=flags)
    else:
        rc = spec_verify(logits_p, logits_q, draft_tokens, u_accept, u_resample, T, tokens, n_acc, workspace,
                         out_logz=logz, out_flags=flags, events=events)
    if rc != 0:
        raise SpecVerifyError(rc, strerror(rc))
    out = (tokens, n_acc)
    if return_logz:
        out += (logz,)
    if return_flags:
        out += (flags,)
    return out


def verify_tree_greedy(logits, tree_tokens, parents, *, workspace=None):
    """Greedy verification of B token trees on torch device tensors.

    logits [B,N,V] (bf16 or fp32), tree_tokens and parents [B,N] int32, all
    contiguous on one device.  Returns (tokens [B,N], path [B,N],
    n_accepted [B]) as int32 device tensors; nothing synchronises."""
    import torch
    dev = logits.device
    if dev.type != "cuda" or logits.dim() != 3:
        raise ValueError("logits must be a [B, N, V] device tensor")
    B, N, V = logits.shape
    for t in (tree_tokens, parents):
        if t.device != dev or t.dtype != torch.int32 or tuple(t.shape) != (B, N) or not t.is_contiguous():
            raise ValueError("tree_tokens and parents must be contiguous int32 [B, N] on the logits' device")
    if not logits.is_contiguous():
        raise ValueError("logits must be contiguous")
    dt = _dtype_code(logits)
    need = int(load().spec_verify_tree_workspace_size(B, N, V, dt))
    if need == 0:
        raise SpecVerifyError(-2, "invalid tree shape")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    rc = int(load().spec_verify_tree_greedy(_ptr(logits), _ptr(tree_tokens), _ptr(parents), B, N, V, _ptr(tokens),
                                            _ptr(path), _ptr(n_acc), dt, _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), st))
    if rc != 0:
        raise SpecVerifyError(rc, strerror(rc))
    return tokens, path, n_acc


def tree_mask(parents):
    """Tree attention mask [B,N,N] uint8 and depth position ids [B,N] int32
    of B trees given by parents [B,N] int32 (a device tensor)."""
    import torch
    if parents.device.type != "cuda" or parents.dtype != torch.int32 or parents.dim() != 2 or \
            not parents.is_contiguous():
        raise ValueError("parents must be a contiguous int32 [B, N] device tensor")
    B, N = parents.shape
    mask = torch.empty((B, N, N), dtype=torch.uint8, device=parents.device)
    depth = torch.empty((B, N), dtype=torch.int32, device=parents.device)
    st = torch.cuda.current_stream(parents.device).cuda_stream
    rc = int(load().spec_tree_mask(_ptr(parents), B, N, _ptr(mask), _ptr(depth), st))
    if rc != 0:
        raise SpecVerifyError(rc, strerror(rc))
    return mask, depth


def ngram_propose(history, lengths, n_min: int, n_max: int, min_hits: int, K: int):
    """Prompt-lookup drafts for B token histories (device tensors: history
    [B, L_max] int32 padded, lengths [B] int32).  Returns (draft [B, K],
    count [B]) int32 device tensors; nothing synchronises."""
    import torch
    dev = history.device
    if dev.type != "cuda" or history.dtype != torch.int32 or history.dim() != 2 or not history.is_contiguous():
        raise ValueError("history must be a contiguous int32 [B, L_max] device tensor")
    B, L = history.shape
    if lengths.device != dev or lengths.dtype != torch.int32 or tuple(lengths.shape) != (B,):
        raise ValueError("lengths must be an int32 [B] tensor on the history's device")
    draft = torch.empty((B, K), dtype=torch.int32, device=dev)
    count = torch.empty((B,), dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    rc = int(load().spec_ngram_propose(_ptr(history), _ptr(lengths), B, L, n_min, n_max, min_hits, K, _ptr(draft),
                                       _ptr(count), st))
    if rc != 0:
        raise SpecVerifyError(rc, strerror(rc))
    return draft, count


NGRAM_MAP_FULL = 1  # SPECV_NGRAM_MAP_FULL


def ngram_map_bytes(B: int, capacity: int) -> int:
    """Device bytes of B n-gram map tables of `capacity` slots (0 if invalid)."""
    return int(load().spec_ngram_map_bytes(B, capacity))


def ngram_map_update(tables, capacity: int, history, len_old, len_new, n_min: int, n_max: int, min_hits: int,
                     K: int):
    """spec_ngram_map_update on device tensors: tables (uint8, ngram_map_bytes
    bytes, kept between calls), history [B, L_max] int32, len_old and len_new
    [B] int32.  Returns (draft [B, K], count [B], status [B]) int32 device
    tensors; nothing synchronises."""
    import torch
    dev = history.device
    if dev.type != "cuda" or history.dtype != torch.int32 or history.dim() != 2 or not history.is_contiguous():
        raise ValueError("history must be a contiguous int32 [B, L_max] device tensor")
    B, L = history.shape
    for name, t in (("len_old", len_old), ("len_new", len_new)):
        if t.device != dev or t.dtype != torch.int32 or tuple(t.shape) != (B,):
            raise ValueError(f"{name} must be an int32 [B] tensor on the history's device")
    if tables.device != dev or tables.numel() * tables.element_size() < ngram_map_bytes(B, capacity):
        raise ValueError("tables must be a device tensor of ngram_map_bytes(B, capacity) bytes")
    draft = torch.empty((B, K), dtype=torch.int32, device=dev)
    count = torch.empty((B,), dtype=torch.int32, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    rc = int(load().spec_ngram_map_update(_ptr(tables), capacity, _ptr(history), _ptr(len_old), _ptr(len_new), B, L,
                                          n_min, n_max, min_hits, K, _ptr(draft), _ptr(count), _ptr(status), st))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_ngram_map_update")
    return draft, count, status


def rounds_min_bytes(bytes_: Optional[float] = None) -> float:
    """The input size from which verify calls read rows in rounds (early
    exit); sets it when bytes_ is given.  Returns the previous value."""
    return float(load().spec_rounds_min_bytes(-1.0 if bytes_ is None else float(bytes_)))


def short_max_seqs(n: Optional[int] = None) -> int:
    """The largest batch whose sampling calls on rows of at most 2048 tokens
    take the one-launch path; sets it when n is given (0: never).  Returns the
    previous value."""
    return int(load().spec_short_max_seqs(-1 if n is None else int(n)))
