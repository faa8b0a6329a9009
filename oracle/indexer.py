"""Lightning-indexer scores (oracle, float64).  Test infrastructure only.

Page: "DeepSeek-V4 deep dive", section 5.2, the scoring equation
I_{s,t} = sum_h w_{s,h} ReLU(q_{s,h} . k_t), with block t visible to the query
at position s iff t < floor((s + 1) / 4); and its implementation notes (the
head weights are pre-scaled by 128**-0.5 * H**-0.5, which the caller folds
into w; the Hadamard rotation applied to q and k leaves every dot product
unchanged).
"""

import numpy as np


def n_visible(pos, ratio, n_max=None):
    """Number of completed compressed blocks a query at ``pos`` may read."""
    n = (np.asarray(pos, dtype=np.int64) + 1) // ratio
    if n_max is not None:
        n = np.minimum(n, n_max)
    return n


def scores(q_idx, w, keys, n_vis):
    """q_idx [H, d], w [H], keys [N, d] (float64 values) -> S [n_vis] float64."""
    q = np.asarray(q_idx, dtype=np.float64)
    K = np.asarray(keys, dtype=np.float64)[:n_vis]
    dots = K @ q.T  # [n_vis, H]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


def scores_loop(q_idx, w, keys, n_vis):
    """Same quantity with explicit per-block, per-head loops (tiny inputs)."""
    out = []
    for t in range(n_vis):
        acc = 0.0
        for h in range(len(w)):
            d = 0.0
            for c in range(len(q_idx[h])):
                d += float(q_idx[h][c]) * float(keys[t][c])
            acc += float(w[h]) * max(d, 0.0)
        out.append(acc)
    return np.array(out)
