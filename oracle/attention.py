"""Index lists and shared-KV multi-query attention with a sink (oracle, float64).

Test infrastructure only.

Pages: "DeepSeek-V4 deep dive"
* section 3.1: one 512-d entry per position is both key and value for every
  query head;
* section 3.3: RoPE on the last 64 dims of the query (and of every entry, as
  stored), and the output's last 64 dims rotated back by the query's own
  position;
* section 3.4, Eq. 27: s = exp(z) / (sum_k exp(z_k) + exp(z'_h)) with
  z = q . c / sqrt(512), o = sum_j s_j c_j; the sink joins the denominator
  only; one softmax over window and compressed rows, duplicates kept;
* section 2.1 notes and 5.3: the list is [128 window ids ; compressed ids],
  the window covers the last 128 positions including the query, padded with
  -1 early in the sequence, and -1 rows are masked out;
* section 6.1: an HCA list holds every completed entry 0 .. floor((t+1)/128)-1.

Readings: the decode window is a 128-slot ring addressed by position mod 128;
the prefill window is addressed linearly (row = position - base); with no
valid row the output is zero.
"""

import numpy as np

from . import rope as _rope

WINDOW = 128


def window_ids(t, mode="ring", base=0, window=WINDOW, n_rows=None):
    """Window row ids for a query at position t (-1 where position < 0).

    ring: row = position mod window; linear: row = position - base, and -1
    when that row falls outside [0, n_rows) (reading: a row the buffer does
    not hold is absent, like a -1 id)."""
    p = t - (window - 1) + np.arange(window)
    if mode == "ring":
        ids = np.where(p >= 0, p % window, -1)
    elif mode == "linear":
        ids = np.where(p >= 0, p - base, -1)
        if n_rows is not None:
            ids = np.where((ids >= 0) & (ids < n_rows), ids, -1)
    else:
        raise ValueError(mode)
    return ids.astype(np.int64)


def hca_ids(t, ratio=128, n_max=None):
    n = (t + 1) // ratio
    if n_max is not None:
        n = min(n, n_max)
    return np.arange(n, dtype=np.int64)


def attend(q, rows, valid, sink, scale, pos, omega):
    """One query unit.

    q     [H, D] un-rotated query (float64 values)
    rows  [n, D] gathered entries in stored (already rotated) form
    valid [n] bool
    sink  [H]
    Returns o' [H, D] (float64) after the inverse rotation.
    """
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    qr = _rope.rotate(q, pos, omega)
    C = np.asarray(rows, dtype=np.float64)[np.asarray(valid, dtype=bool)]
    sink = np.asarray(sink, dtype=np.float64)
    if C.shape[0] == 0:
        return np.zeros((H, D))
    z = (qr @ C.T) * scale  # [H, n]
    m = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - m)
    den = np.sum(e, axis=1) + np.exp(sink - m[:, 0])
    o = (e @ C) / den[:, None]
    return _rope.rotate(o, pos, omega, inverse=True)


def sparse_decode(q, win_rows, win_valid_ids, entries, topk_ids, sink, scale, pos, omega):
    """CSA: list = window ids then top-k ids (compressed space), -1 = none."""
    wid = np.asarray(win_valid_ids)
    tid = np.asarray(topk_ids)
    rows = []
    valid = []
    for i in wid:
        rows.append(win_rows[i] if i >= 0 else np.zeros(q.shape[-1]))
        valid.append(i >= 0)
    for i in tid:
        rows.append(entries[i] if i >= 0 else np.zeros(q.shape[-1]))
        valid.append(i >= 0)
    return attend(q, np.array(rows), np.array(valid), sink, scale, pos, omega)


def hca_decode(q, win_rows, win_ids, entries, sink, scale, pos, omega, ratio=128):
    ids = hca_ids(pos, ratio, n_max=entries.shape[0])
    return sparse_decode(q, win_rows, win_ids, entries, ids, sink, scale, pos, omega)
