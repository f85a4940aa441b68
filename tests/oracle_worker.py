"""Worker functions that run oracle pieces in separate processes.

Imports only numpy and the oracle, so a spawned worker starts fast.
"""

import numpy as np

import oracle as U


def segment_prefill_oracle(args):
    """Final log-biases and sampled outputs of one prefill segment.

    The oracle's dense definitions (O5 as column sums, O7 per row) on the
    GPU-stored keys; returns (final Lambda [N], y [len(rows), G, d]).
    """
    (terms, Kt, V, lq, lk, lb, q_rows, gam_rows, rows, scale, base) = args
    N = Kt.shape[0]
    lam_rows = U.dense_logbias(terms, Kt, lq, lk, lb, rows=np.append(rows, N - 1))
    ys = []
    for ri, i in enumerate(rows):
        qt = U.rope(q_rows[ri], np.full(q_rows.shape[1], i), base)
        ys.append(gam_rows[ri] * U.attend(qt, Kt[: i + 1], V[: i + 1], lam_rows[ri, : i + 1], scale))
    return lam_rows[-1], np.stack(ys)
