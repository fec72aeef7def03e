"""The per-token upstream weights (dloss) of the synthetic cases, from the oracle.

The generators in ``synth`` name the reduction a case stands for and leave
its weights to the caller; the tests take them from ``oracle.loss_weights``
(the token mean, m / max(sum m, 1)) or, for the plain sum of the per-token
losses, the completion mask itself (weight 1 on every kept token).
"""
import numpy as np

import oracle


def fill_dloss(case):
    """Set ``case.dloss`` (fp32 [B*L]) for ``case.dloss_kind``; returns the case."""
    if case.dloss is None:
        if case.dloss_kind == "mean":
            w = oracle.loss_weights(case.mask, case.B, case.L, "token")
        elif case.dloss_kind == "sum":
            w = (np.asarray(case.mask) != 0).astype(np.float64)
        else:
            raise ValueError(f"case {case.name}: no weights for {case.dloss_kind!r}")
        case.dloss = w.astype(np.float32)
    return case
