"""Block cache and per-request state slots of a decode server (oracle, plain
index arithmetic).  Test infrastructure only (see the package docstring).

Page: "DeepSeek-V4 deep dive", section 9.4 (Serving the heterogeneous cache):
* compressed entries live in a block cache whose blocks each cover a multiple
  of lcm(4, 128) = 128 original tokens: for one 128-token block a CSA layer
  stores 32 entries (and their index keys), an HCA layer one entry;
* everything still in motion lives in one fixed-size state slot per request,
  drawn from a pre-allocated pool: the window's last 128 rows and the
  uncompressed tail (tokens that do not fill a block yet; for the
  overlapping ratio-4 compressor also the previous block it reuses);
* the worked example: a 1,000-token prompt gives 250 CSA entries and 7 HCA
  entries, a window of tokens 872 .. 999, 104 pending tokens per HCA layer,
  and, per CSA layer, only the last 4-token block.

Readings (listed in the design notes): a request's blocks are found through a
block table, row b listing the pool block of each logical block j of
sequence b (-1: not allocated), so logical entry e sits at row e mod bs of
pool block table[b][e // bs], bs = 128 // ratio; the state slot of sequence
b is slot[b] in the pool of slots.
"""

import math

import numpy as np

WINDOW = 128


def tokens_per_block(ratios=(4, 128)):
    """A block covers lcm of the compression ratios: 128 tokens for V4."""
    return math.lcm(*ratios)


def entries_per_block(ratio, tokens=None):
    """Compressed entries (and, for CSA, index keys) in one block."""
    tokens = tokens_per_block() if tokens is None else tokens
    assert tokens % ratio == 0
    return tokens // ratio


def layer_blocks(n_tokens, ratio):
    """(completed entries, blocks they occupy) after n_tokens tokens."""
    n = n_tokens // ratio
    bs = entries_per_block(ratio)
    return n, -(-n // bs)


def state_slot(n_tokens, ratio, window=WINDOW):
    """What the request's state slot holds after n_tokens tokens, as token
    positions: the window (first, last), the pending tail (first, last) or
    None, and for ratio 4 the previous block reused by the overlap."""
    first = max(0, n_tokens - window)
    done = (n_tokens // ratio) * ratio
    out = {"window": (first, n_tokens - 1),
           "pending": (done, n_tokens - 1) if done < n_tokens else None}
    if ratio == 4:
        out["overlap"] = (done - ratio, done - 1) if done >= ratio else None
    return out


def entry_address(table, bs, e):
    """(pool block, row in block) of logical entry e, or None when e < 0 or
    its block is not allocated."""
    if e < 0 or e // bs >= len(table):
        return None
    blk = int(table[e // bs])
    if blk < 0:
        return None
    return blk, e % bs


def scatter(entries, table, bs, n_blocks):
    """A pool [n_blocks, bs, row] holding entries [N, row] at their table
    addresses (rows of unallocated or unused slots stay zero)."""
    entries = np.asarray(entries)
    pool = np.zeros((n_blocks, bs) + entries.shape[1:], dtype=entries.dtype)
    for e in range(entries.shape[0]):
        a = entry_address(table, bs, e)
        if a is not None:
            pool[a] = entries[e]
    return pool


def gather(pool, table, bs, ids):
    """Rows of logical entries ids (an absent id gives a zero row) and a
    validity mask."""
    rows = np.zeros((len(ids),) + pool.shape[2:], dtype=pool.dtype)
    valid = np.zeros(len(ids), dtype=bool)
    for j, e in enumerate(ids):
        a = entry_address(table, bs, int(e))
        if a is not None:
            rows[j] = pool[a]
            valid[j] = True
    return rows, valid


def allocate(entries_per_seq, bs, n_blocks, rng, max_blocks=None):
    """Block tables [B, max_blocks] of distinct pool blocks for sequences of
    the given entry counts, drawn at random from a pool of n_blocks (-1 past
    each sequence's last block)."""
    need = [-(-int(n) // bs) for n in entries_per_seq]
    max_blocks = max(need) if max_blocks is None else max_blocks
    assert sum(need) <= n_blocks and max(need) <= max_blocks
    perm = rng.permutation(n_blocks)
    table = np.full((len(need), max_blocks), -1, dtype=np.int32)
    k = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[k:k + nb]
        k += nb
    return table
