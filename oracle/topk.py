"""Deterministic top-k selection (oracle).  Test infrastructure only.

Page: "DeepSeek-V4 deep dive", section 5.2 step 5 (the selector keeps
min(k, number of visible blocks) entries) and section 3.4 / 5.3 notes
(padding ids are -1).

Reading for what the pages leave open (listed in the design notes): the
output is ordered by descending score, equal scores go to the smaller index
first, -0.0 equals +0.0, and NaN ranks below every number (NaNs among
themselves by index).  The worked example of section 5.3 lists the chosen
blocks in descending-score order, which this follows.  For the bit-exact
comparison the scores are compared as given (float32).
"""

import numpy as np


def _order(scores):
    s = np.asarray(scores)
    v = s.astype(np.float64)
    nan = np.isnan(v)
    v = np.where(nan, 0.0, v) + 0.0  # -0.0 -> +0.0
    idx = np.arange(len(s))
    # lexsort: last key is primary -> (nan last, value desc, index asc)
    return np.lexsort((idx, -v, nan.astype(np.int8)))


def topk(scores, k, n_vis=None):
    """Indices (int32 [k]) of the top min(k, n_vis) scores, -1 padded."""
    s = np.asarray(scores)
    n = len(s) if n_vis is None else int(n_vis)
    out = np.full(k, -1, dtype=np.int32)
    if n <= 0 or k <= 0:
        return out
    o = _order(s[:n])[:min(k, n)]
    out[:len(o)] = o
    return out


def topk_bruteforce(scores, k, n_vis=None):
    """Repeated arg-best with explicit comparisons (tiny inputs only)."""
    s = [float(x) for x in scores]
    n = len(s) if n_vis is None else int(n_vis)

    def better(i, j):  # does i rank before j?
        a, b = s[i], s[j]
        if a != a:  # NaN
            return (b != b) and i < j
        if b != b:
            return True
        if a != b:
            return a > b
        return i < j

    taken = set()
    out = []
    for _ in range(min(k, n)):
        best = None
        for i in range(n):
            if i in taken:
                continue
            if best is None or better(i, best):
                best = i
        taken.add(best)
        out.append(best)
    return np.array(out + [-1] * (k - len(out)), dtype=np.int32)
