"""The whole CSA decode path for one sequence, from hidden states (oracle).

Test infrastructure only.  Composes the other oracle modules in the order of
"DeepSeek-V4 deep dive" section 5.1 (compress main KV, compress index keys,
score and select, attend over window + selection in one softmax) and
section 3.4 (the list layout).
"""

import numpy as np

from . import attention, codec, compressor, indexer, topk as _topk


def compress_all(x, start_pos, wkv, wgate, ape, norm_w, omega, ratio, head_dim, rotate,
                 store_fmt, n_entries, state=None):
    """Run the (bulk) compressor and return the stored entries as float64."""
    out, st = compressor.compress_bulk(x, start_pos, wkv, wgate, ape, norm_w, omega, ratio,
                                       head_dim, rotate=rotate, state=state)
    E = np.zeros((n_entries, head_dim))
    for i, v in out.items():
        if i < n_entries:
            E[i] = codec.store(v, store_fmt)[1]
    return E, st


def csa_decode_from_hidden(x, main, idx, q, q_idx, w_idx, sink, win_rows, t, k, omega,
                           ent_fmt="f32", key_fmt="f32", scale=512 ** -0.5, ratio=4):
    """x [T, dim] covers positions 0..T-1 and the query sits at t = T - 1.

    main / idx: dicts with wkv, wgate, ape, norm_w for the 512-wide main
    compressor and the 128-wide (rotated) indexer compressor.
    Returns a dict of entries, keys, scores, topk ids and the output [H, 512].
    """
    n = (t + 1) // ratio
    E, _ = compress_all(x, 0, main["wkv"], main["wgate"], main["ape"], main["norm_w"], omega,
                        ratio, 512, False, ent_fmt, n)
    K, _ = compress_all(x, 0, idx["wkv"], idx["wgate"], idx["ape"], idx["norm_w"], omega,
                        ratio, 128, True, key_fmt, n)
    S = indexer.scores(q_idx, w_idx, K, n)
    sel = _topk.topk(S.astype(np.float32), k, n)
    wid = attention.window_ids(t)
    o = attention.sparse_decode(q, win_rows, wid, E, sel, sink, scale, t, omega)
    return {"entries": E, "keys": K, "scores": S, "topk": sel, "out": o}
