"""GPU-side helpers of the parity tests: run the HIP path on a batch."""
import numpy as np

import workloads
from oracle.parity import GpuOut


def run_gpu(sv, batch, dev_inputs=None, position_stats=None) -> GpuOut:
    """The HIP path on a batch, with log Z (sampling mode) and flags; a batch
    with per-sequence draft counts goes through spec_verify_ragged_ex."""
    import torch
    lp, lq, x, ua, ur = dev_inputs if dev_inputs is not None else workloads.to_device(batch)
    greedy = batch.T == 0.0
    nd = getattr(batch, "num_drafts", None)
    kb = None
    if nd is not None:
        kb = torch.from_numpy(np.ascontiguousarray(nd, dtype=np.int32)).to(lp.device)
    out = sv.verify(lp, lq, x, ua, ur, batch.T, return_logz=not greedy, return_flags=True, num_drafts=kb,
                    position_stats=position_stats)
    torch.cuda.synchronize()
    if greedy:
        tok, n, flags = out
        logz = None
    else:
        tok, n, logz, flags = out
        logz = logz.cpu().numpy()
    return GpuOut(tok.cpu().numpy(), n.cpu().numpy(), logz, flags.cpu().numpy())


