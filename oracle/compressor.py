"""Learned gated-pooling KV compressor (oracle, float64).  Test infrastructure only.

Pages: "DeepSeek-V4 deep dive", section 4.1 (the pooling equation:
s_j = W_gate x_j + B_{j mod r}, v_j = W_kv x_j, C_{i,c} = sum_j softmax_j(s_{j,c})
v_{j,c}), section 4.2 (ratio 4 overlaps with the previous block through the
first half of a doubled projection; ratio 128 does not; post-processing
RMSNorm -> RoPE at the block's first position -> storage rounding; emission
when (p+1) mod r == 0), section 4.3 notes (decode state: kv/score slots,
score initialised to -inf, shift of the current block into the previous
slots), and section 5.2 (the indexer's own ratio-4 compressor, 128 wide, with
a Hadamard rotation after RoPE).

Two independent implementations are given and must agree exactly in float64:

* ``compress_bulk`` builds, for every block completed by the call, the 2r- or
  r-slot pooling window from a position-indexed table of projections
  (section 4.2 steps 1-4), and
* ``compress_stream`` feeds one token at a time through the slot state
  machine of the decode path (section 4.3 notes).

Readings (listed in the design notes): RMSNorm eps = 1e-6 and form
x / sqrt(mean(x^2) + eps) * g; compressor input is used as given; the entry of
block i is rotated at position i * r, also for overlapped entries; the
Hadamard matrix is Sylvester's H_128 scaled by 128**-0.5; ratio 1 (tests only)
pools a single slot, so the entry is the projection itself.
"""

import numpy as np

from . import rope as _rope

NEG_INF = -np.inf


def coff_of(ratio):
    """Projection width multiplier: 2 when the ratio-4 overlap is used."""
    return 2 if ratio == 4 else 1


def hadamard(n):
    """Sylvester Hadamard matrix H_n (n a power of two), entries +-1."""
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == n
    return H


def rmsnorm(x, g, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def postprocess(C, block_index, ratio, norm_w, omega, rotate, eps=1e-6):
    """RMSNorm -> RoPE at position block_index*ratio -> optional Hadamard.

    Storage rounding is applied by the caller with ``codec.store``.
    """
    d = C.shape[-1]
    y = rmsnorm(C, norm_w, eps)
    y = _rope.rotate(y, np.asarray(block_index) * ratio, omega)
    if rotate:
        y = y @ (hadamard(d).T / np.sqrt(d))
    return y


def empty_state(ratio, head_dim):
    """(kv_state, score_state), each [coff*r, coff*d]; score starts at -inf."""
    co = coff_of(ratio)
    kv = np.zeros((co * ratio, co * head_dim))
    sc = np.full((co * ratio, co * head_dim), NEG_INF)
    return kv, sc


def project(x, w_kv, w_gate, ape, positions, ratio):
    """v = W_kv x and s = W_gate x + ape[p mod r] for each token (rows)."""
    x = np.asarray(x, dtype=np.float64)
    v = x @ np.asarray(w_kv, dtype=np.float64).T
    s = x @ np.asarray(w_gate, dtype=np.float64).T + np.asarray(ape, dtype=np.float64)[
        np.asarray(positions) % ratio]
    return v, s


def _pool(v_slots, s_slots):
    """Per-channel softmax over the slot axis, then the weighted sum."""
    m = np.max(s_slots, axis=0)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s_slots - m)
    return np.sum(e * v_slots, axis=0) / np.sum(e, axis=0)


def compress_stream(x, start_pos, w_kv, w_gate, ape, norm_w, omega, ratio, head_dim,
                    rotate=False, state=None, eps=1e-6):
    """Token-at-a-time state machine.  Returns ({entry_index: vector}, state)."""
    co = coff_of(ratio)
    d = head_dim
    kv, sc = empty_state(ratio, d) if state is None else (state[0].copy(), state[1].copy())
    out = {}
    T = x.shape[0]
    for j in range(T):
        p = start_pos + j
        v, s = project(x[j:j + 1], w_kv, w_gate, ape, [p], ratio)
        slot = (ratio if co == 2 else 0) + p % ratio
        kv[slot] = v[0]
        sc[slot] = s[0]
        if (p + 1) % ratio == 0:
            i = p // ratio
            if co == 2:
                vs = np.concatenate([kv[:ratio, :d], kv[ratio:, d:]], axis=0)
                ss = np.concatenate([sc[:ratio, :d], sc[ratio:, d:]], axis=0)
            else:
                vs, ss = kv, sc
            C = _pool(vs, ss)
            out[i] = postprocess(C, i, ratio, norm_w, omega, rotate, eps)
            if co == 2:
                kv[:ratio] = kv[ratio:]
                sc[:ratio] = sc[ratio:]
    return out, (kv, sc)


def compress_bulk(x, start_pos, w_kv, w_gate, ape, norm_w, omega, ratio, head_dim,
                  rotate=False, state=None, eps=1e-6):
    """Window build over a position-indexed projection table.

    Every block whose last token lies in this call is pooled from the table,
    where positions before ``start_pos`` are read from the incoming state.
    Returns ({entry_index: vector}, new state) like ``compress_stream``.
    """
    co = coff_of(ratio)
    d = head_dim
    T = x.shape[0]
    p0 = start_pos
    p1 = start_pos + T  # exclusive
    kv0, sc0 = empty_state(ratio, d) if state is None else state
    pos = np.arange(p0, p1)
    v_new, s_new = project(x, w_kv, w_gate, ape, pos, ratio)

    # position -> (v, s) table for everything the call can need
    table = {}
    cur_block = p0 // ratio
    # incoming state: current-block slots hold positions cur_block*r .. p0-1
    for p in range(cur_block * ratio, p0):
        slot = (ratio if co == 2 else 0) + p % ratio
        table[p] = (kv0[slot], sc0[slot])
    # previous-block slots (overlap only) hold the block before cur_block
    if co == 2 and cur_block >= 1:
        for a in range(ratio):
            table[(cur_block - 1) * ratio + a] = (kv0[a], sc0[a])
    for j, p in enumerate(pos):
        table[int(p)] = (v_new[j], s_new[j])

    def get(p):
        if p < 0:
            return np.zeros(co * d), np.full(co * d, NEG_INF)
        return table[p]

    out = {}
    first_block = p0 // ratio
    last_block = p1 // ratio - 1  # last block completed by this call
    for i in range(first_block, last_block + 1):
        if (i + 1) * ratio - 1 < p0:
            continue
        if co == 2:
            prev = [get(i * ratio - ratio + a) for a in range(ratio)]
            curr = [get(i * ratio + a) for a in range(ratio)]
            vs = np.stack([t[0][:d] for t in prev] + [t[0][d:] for t in curr])
            ss = np.stack([t[1][:d] for t in prev] + [t[1][d:] for t in curr])
        else:
            blk = [get(i * ratio + a) for a in range(ratio)]
            vs = np.stack([t[0] for t in blk])
            ss = np.stack([t[1] for t in blk])
        out[i] = postprocess(_pool(vs, ss), i, ratio, norm_w, omega, rotate, eps)

    # new state: current slots = the unfinished block's tokens; stale slots are
    # left as they were.  Previous slots = last completed block (overlap).
    kv, sc = kv0.copy(), sc0.copy()
    end_block = p1 // ratio  # block holding position p1 (unfinished)
    for p in range(max(end_block * ratio, p0), p1):
        slot = (ratio if co == 2 else 0) + p % ratio
        kv[slot], sc[slot] = table[p]
    if end_block > first_block:
        # a block completed in this call: the decode state machine shifts the
        # current slots into the previous ones (overlap) and never resets a
        # slot, so every slot not yet rewritten holds the last completed block
        done = end_block - 1
        for a in range(ratio):
            if co == 2:
                kv[a], sc[a] = get(done * ratio + a)
                kv[ratio + a], sc[ratio + a] = get(done * ratio + a)
            else:
                kv[a], sc[a] = get(done * ratio + a)
        for p in range(end_block * ratio, p1):
            slot = (ratio if co == 2 else 0) + p % ratio
            kv[slot], sc[slot] = table[p]
    return out, (kv, sc)
