"""The whole CSA decode path for one sequence, from hidden states (oracle).

Test infrastructure only.  Composes the other oracle modules in the order of
"DeepSeek-V4 deep dive" section 5.1 (compress main KV, compress index keys,
score and select, attend over window + selection in one softmax) and
section 3.4 (the list layout); ``layer_decode_step`` adds the layer's steps
on either side (sections 3.2, 3.3, 3.5, 5.2): the query path, index queries
and weights and the window-entry write before the path, the grouped output
projection after it.
"""

import numpy as np

from . import attention, codec, compressor, indexer, layer, topk as _topk


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


def layer_decode_step(x, t, wts, ring, win_fmt, entries, keys, sink, k, omega,
                      scale=512 ** -0.5, ratio=4, ids=None, eps=1e-6):
    """One decode step of a CSA layer for the token at position t.

    x        [dim] the token's hidden state
    wts      layer weights (``layer.layer_input`` / ``layer.output_projection``
             keys, plus H and Hi)
    ring     [128, 512] the window ring's stored values before the step
    entries  [N, 512], keys [N, 128]: stored values of the compressed cache,
             including whatever the compressor emitted at this step
    ids      the top-k list to attend over, as row ids of ``entries``; None
             selects with the oracle's own scores over the keys

    The query heads go into attention before RoPE; attention rotates them at
    t once (section 3.3: q and k each carry the rotation of their own
    position).  Returns a dict of q (pre-RoPE), q_idx, w_idx, the window
    entry (before rounding), the ring after the write, scores, topk, the
    attention output o and the layer output y.
    """
    q, qi, wi, kv = layer.layer_input(x, t, wts, omega, eps, rotate_q=False)
    ring = layer.window_write(ring, codec.store(kv, win_fmt)[1], t)
    n = int(indexer.n_visible(t, ratio, keys.shape[0]))
    S = indexer.scores(qi, wi, keys, n)
    sel = _topk.topk(S.astype(np.float32), k, n)
    use = sel if ids is None else np.asarray(ids)
    o = attention.sparse_decode(q, ring, attention.window_ids(t), entries, use, sink, scale, t,
                                omega)
    y = layer.output_projection(o, wts["wo_a"], wts["wo_b"])
    return {"q": q, "q_idx": qi, "w_idx": wi, "kv": kv, "ring": ring, "scores": S, "topk": sel,
            "out": o, "y": y}
