"""libspecverify: the verify step of speculative sampling on MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C ABI
(include/specverify.h); this package is a thin ctypes binding over it.
"""
from ._lib import (DEBUG_COUNTERS, ERRORS, EXPORTS, FLAG_BAD_DRAFT, FLAG_FP64, FLAG_ZW_ZERO, LIB_PATH, NOALLOC_SCRATCH, SPECV_BF16,
                   SPECV_F32, SPECV_MAX_K, SPECV_MAX_NGRAM, SPECV_MAX_TREE, SpecVerifyError, bind_spec_verify,
                   bind_spec_verify_ragged, debug_counters, debug_enable, debug_reset, load, NGRAM_MAP_FULL,
                   ngram_map_bytes, ngram_map_update, ngram_propose, rounds_min_bytes, short_max_seqs,
                   spec_verify, spec_verify_noalloc, spec_verify_ragged, spec_verify_sweep_timed, strerror,
                   tree_mask, verify,
                   verify_tree_greedy, version, workspace_size)

__all__ = ["DEBUG_COUNTERS", "ERRORS", "EXPORTS", "FLAG_BAD_DRAFT", "FLAG_FP64", "FLAG_ZW_ZERO", "LIB_PATH", "SPECV_BF16", "SPECV_F32",
           "SPECV_MAX_K", "SPECV_MAX_NGRAM", "SPECV_MAX_TREE", "NOALLOC_SCRATCH", "SpecVerifyError",
           "bind_spec_verify", "bind_spec_verify_ragged", "debug_counters", "debug_enable", "debug_reset", "load",
           "NGRAM_MAP_FULL", "ngram_map_bytes", "ngram_map_update", "ngram_propose", "rounds_min_bytes", "short_max_seqs", "spec_verify", "spec_verify_noalloc", "spec_verify_ragged", "spec_verify_sweep_timed",
           "strerror", "tree_mask", "verify", "verify_tree_greedy", "version", "workspace_size"]
