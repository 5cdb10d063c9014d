"""GPU-side helpers of the parity tests: run the HIP path on a batch."""
import numpy as np

import workloads
from oracle.parity import GpuOut


def run_gpu(sv, batch, dev_inputs=None, position_stats=None) -> GpuOut:
    """The HIP path on a batch, both ways the library sweeps:

    * the product path (no log Z asked for): rows past a sequence's first
      rejection are not read;
    * with every row's log Z asked for: one sweep of every row.

    Both must give bit-identical tokens, counts and flags (each chunk's
    partial is computed by the same code either way).  Returns the product
    path's tokens, counts and flags with the full sweep's log Z.  A batch with
    per-sequence draft counts goes through spec_verify_ragged(_ex); position
    counters, when given, are added by the product call only."""
    import torch
    lp, lq, x, ua, ur = dev_inputs if dev_inputs is not None else workloads.to_device(batch)
    greedy = batch.T == 0.0
    nd = getattr(batch, "num_drafts", None)
    kb = None
    if nd is not None:
        kb = torch.from_numpy(np.ascontiguousarray(nd, dtype=np.int32)).to(lp.device)
    tok, n, flags = sv.verify(lp, lq, x, ua, ur, batch.T, return_flags=True, num_drafts=kb,
                              position_stats=position_stats)
    # with log Z asked for (greedy leaves it untouched, but still sweeps every row)
    tok_f, n_f, logz, flags_f = sv.verify(lp, lq, x, ua, ur, batch.T, return_logz=True, return_flags=True,
                                          num_drafts=kb)
    torch.cuda.synchronize()
    out = GpuOut(tok.cpu().numpy(), n.cpu().numpy(), None if greedy else logz.cpu().numpy(), flags.cpu().numpy())
    np.testing.assert_array_equal(tok_f.cpu().numpy(), out.tokens, err_msg="full sweep vs early exit: tokens")
    np.testing.assert_array_equal(n_f.cpu().numpy(), out.n, err_msg="full sweep vs early exit: counts")
    # the FP64 bit may differ between identical calls where the draw is split
    # over workgroups (batches of at most 128; see SPECV_FLAG_FP64)
    mask = ~0 if len(out.n) > 128 else ~sv.FLAG_FP64
    np.testing.assert_array_equal(flags_f.cpu().numpy() & mask, out.flags & mask,
                                  err_msg="full sweep vs early exit: flags")
    return out
