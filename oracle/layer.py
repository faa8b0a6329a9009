"""The steps of a CSA/HCA attention layer on either side of the decode path
(oracle, float64).  Test infrastructure only (see the package docstring).

Pages: "DeepSeek-V4 deep dive",
  section 3.2 (the query path: wq_a -> q_norm -> wq_b -> per-head RMS rescale
    without a weight; the window entry: wkv -> kv_norm; parameter counts in
    its implementation notes),
  section 3.3 (partial RoPE on the last 64 dims of every query head and of the
    window entry, at the token's own position; the window rows' storage
    precision in its notes),
  section 3.5 (grouped low-rank output projection: g groups of 8 consecutive
    heads, wo_a per group from 8*512 to o_rank, concatenation, wo_b to the
    hidden size; the parameter table),
  section 5.2 (index queries: the shared latent qr through the indexer's own
    wq_b to Hi heads of 128, RoPE on the last 64, Hadamard rotation; head
    weights weights_proj(x) * 128**-0.5 * Hi**-0.5),
  section 3.4 notes (decode window: a 128-slot ring, position p in slot
    p mod 128).

Readings (listed in the design notes):
* RMSNorm is x / sqrt(mean(x^2) + eps) * g with eps = 1e-6, also for the
  weightless per-head rescale (g = 1).
* The latent qr and the grouped projection's intermediate are held in bf16
  between the two matrix products, the precision the pages' code keeps its
  activations in; both are rounded once, to nearest even.
* The window entry is stored in the window ring's row format by the codec
  (``codec.store``); the pages' mixed FP8/bf16 simulation is not a stored
  format here.
* The Hadamard matrix is Sylvester's H_128 scaled by 128**-0.5, as for the
  index keys.
"""

import numpy as np

from . import codec as _codec
from . import compressor as _comp
from . import rope as _rope

HEAD_DIM = 512
INDEX_DIM = 128
WINDOW = 128
GROUP_HEADS = 8


def rmsnorm(x, g=1.0, eps=1e-6):
    """x / sqrt(mean(x^2) + eps) * g over the last axis (section 3.2)."""
    return _comp.rmsnorm(x, g, eps)


def latent(x, wq_a, q_norm, eps=1e-6):
    """qr = q_norm(wq_a x), rounded to bf16 (section 3.2 steps 1-2)."""
    c = np.asarray(x, dtype=np.float64) @ np.asarray(wq_a, dtype=np.float64).T
    return _codec.round_to_bf16(rmsnorm(c, q_norm, eps))


def query_heads(qr, wq_b, H, eps=1e-6):
    """q [..., H, 512] before RoPE: wq_b qr per head, each head divided by its
    own RMS, no weight (section 3.2 steps 3-4).  This is the form the
    attention step takes: it rotates the query at its own position."""
    q = np.asarray(qr, dtype=np.float64) @ np.asarray(wq_b, dtype=np.float64).T
    q = q.reshape(q.shape[:-1] + (H, HEAD_DIM))
    return rmsnorm(q, 1.0, eps)


def queries(qr, wq_b, H, pos, omega, eps=1e-6):
    """q [..., H, 512]: the query heads with RoPE on the last 64 dims at pos
    (sections 3.2 steps 3-4, 3.3)."""
    p = np.asarray(pos)[..., None]
    return _rope.rotate(query_heads(qr, wq_b, H, eps), p, omega)


def index_queries(qr, wq_b_idx, Hi, pos, omega):
    """q_idx [..., Hi, 128]: the indexer's wq_b on the shared latent, RoPE on
    the last 64 dims at pos, then the Hadamard rotation (section 5.2 step 2)."""
    q = np.asarray(qr, dtype=np.float64) @ np.asarray(wq_b_idx, dtype=np.float64).T
    q = q.reshape(q.shape[:-1] + (Hi, INDEX_DIM))
    q = _rope.rotate(q, np.asarray(pos)[..., None], omega)
    return q @ (_comp.hadamard(INDEX_DIM).T / np.sqrt(INDEX_DIM))


def index_weights(x, w_proj):
    """w [..., Hi] = weights_proj(x) * 128**-0.5 * Hi**-0.5 (section 5.2 step 3)."""
    w_proj = np.asarray(w_proj, dtype=np.float64)
    Hi = w_proj.shape[0]
    return (np.asarray(x, dtype=np.float64) @ w_proj.T) * (INDEX_DIM ** -0.5 * Hi ** -0.5)


def window_entry(x, wkv, kv_norm, pos, omega, eps=1e-6):
    """kv [..., 512] = kv_norm(wkv x), RoPE on the last 64 dims at pos
    (sections 3.2 step 5, 3.3)."""
    kv = np.asarray(x, dtype=np.float64) @ np.asarray(wkv, dtype=np.float64).T
    kv = rmsnorm(kv, kv_norm, eps)
    return _rope.rotate(kv, pos, omega)


def window_write(ring, stored_row, pos):
    """The decode window ring with position pos's row in slot pos mod 128
    (section 3.4 notes); ring: [128, row] of stored rows, returned as a copy."""
    out = np.array(ring, copy=True)
    if pos >= 0:
        out[pos % WINDOW] = stored_row
    return out


def output_projection(o, wo_a, wo_b):
    """Grouped low-rank output projection (section 3.5).

    o: [..., H, 512]; wo_a: [g, o_rank, 8*512] (one slice per group of 8
    consecutive heads); wo_b: [dim, g*o_rank].  Group k's 4,096 values go
    through its own slice of wo_a; the g results are concatenated (held in
    bf16) and mapped by wo_b."""
    o = np.asarray(o, dtype=np.float64)
    wo_a = np.asarray(wo_a, dtype=np.float64)
    g, r, w = wo_a.shape
    H = o.shape[-2]
    assert H % g == 0 and (H // g) * HEAD_DIM == w
    og = o.reshape(o.shape[:-2] + (g, w))
    parts = [og[..., k, :] @ wo_a[k].T for k in range(g)]
    mid = _codec.round_to_bf16(np.concatenate(parts, axis=-1))
    return mid @ np.asarray(wo_b, dtype=np.float64).T


def param_counts(dim, q_rank, H, groups, o_rank, Hi=0):
    """Weights per layer implied by the shapes above (section 3.2 notes,
    section 3.5 table, section 5.2 notes)."""
    wq_a = dim * q_rank
    wq_b = q_rank * H * HEAD_DIM
    wkv = dim * HEAD_DIM
    wo_a = groups * o_rank * (H // groups) * HEAD_DIM
    wo_b = groups * o_rank * dim
    return {
        "wq_a": wq_a, "wq_b": wq_b, "wkv": wkv, "wo_a": wo_a, "wo_b": wo_b,
        "grouped_total": wo_a + wo_b, "dense_output": H * HEAD_DIM * dim,
        "wq_b_idx": q_rank * Hi * INDEX_DIM, "weights_proj": dim * Hi,
    }


def layer_input(x, pos, wts, omega, eps=1e-6, rotate_q=True):
    """Everything a decode step needs from the token's hidden state x:
    (q, q_idx or None, w_idx or None, window entry before storage rounding).
    q is the page's rotated query; with rotate_q=False it is the query heads
    before RoPE, the form the attention step takes."""
    qr = latent(x, wts["wq_a"], wts["q_norm"], eps)
    if rotate_q:
        q = queries(qr, wts["wq_b"], wts["H"], pos, omega, eps)
    else:
        q = query_heads(qr, wts["wq_b"], wts["H"], eps)
    kv = window_entry(x, wts["wkv"], wts["kv_norm"], pos, omega, eps)
    if wts.get("Hi", 0):
        qi = index_queries(qr, wts["wq_b_idx"], wts["Hi"], pos, omega)
        wi = index_weights(x, wts["w_proj"])
        return q, qi, wi, kv
    return q, None, None, kv
