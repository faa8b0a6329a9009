"""Pins of the oracle's block cache and state slots (oracle/paged.py), CPU.

* The 1,000-token example of "DeepSeek-V4 deep dive" section 9.4 (fixture
  block_cache_prompt1000): block size, entries per block, entry counts, the
  window and the pending tails.
* The state slot's contents against the compressor oracle's streaming state
  (section 4.3): a state rebuilt from only the tokens the slot is said to
  hold continues the stream exactly as the full state does, and one token
  fewer does not.
* Scatter through random block tables and gather back is the identity on
  the allocated entries; an absent id or block reads as absent.
"""

import numpy as np

from oracle import compressor as CP
from oracle import paged as P
from oracle import rope as R


def test_prompt1000_counts(golden):
    g = golden["block_cache_prompt1000"]
    assert P.tokens_per_block((g["csa_ratio"], g["hca_ratio"])) == g["tokens_per_block"]
    assert P.entries_per_block(g["csa_ratio"]) == g["csa_entries_per_block"]
    assert P.entries_per_block(g["hca_ratio"]) == g["hca_entries_per_block"]
    n, blocks = P.layer_blocks(g["tokens"], g["csa_ratio"])
    assert n == g["csa_entries"] and blocks == 8            # 7 full blocks and one of 26
    n, blocks = P.layer_blocks(g["tokens"], g["hca_ratio"])
    assert n == g["hca_entries"] and blocks == g["hca_entries"]
    s = P.state_slot(g["tokens"], g["hca_ratio"])
    assert s["window"] == (g["window_first"], g["window_last"])
    assert s["pending"][1] - s["pending"][0] + 1 == g["hca_pending_tokens"]
    s = P.state_slot(g["tokens"], g["csa_ratio"])
    assert s["pending"] is None
    assert s["overlap"][1] - s["overlap"][0] + 1 == g["csa_overlap_block_tokens"]
    assert s["overlap"] == (996, 999)


def test_state_slot_holds_all_the_stream_needs():
    """The slot's stated contents are all the compressor's streaming state
    needs: after a 1,000-token prompt, a state rebuilt from only those
    tokens (the last complete 4-token block for ratio 4, the 104 pending
    tokens for ratio 128, every other slot empty) continues the stream to the
    entries the full state gives, up to the float64 rounding of a projection
    taken over a batch of tokens instead of one."""
    rng = np.random.default_rng(3)
    dim, T, more = 8, 1000, 300
    x = rng.standard_normal((T + more, dim))
    om = R.frequencies(160000.0)
    for ratio, d in ((4, 64), (128, 64)):
        co = CP.coff_of(ratio)
        wkv = rng.standard_normal((co * d, dim))
        wg = rng.standard_normal((co * d, dim))
        ape = rng.standard_normal((ratio, co * d))
        args = (wkv, wg, ape, np.ones(d), om, ratio, d)
        _, full = CP.compress_stream(x[:T], 0, *args)
        slot = P.state_slot(T, ratio)
        kv, sc = CP.empty_state(ratio, d)
        if ratio == 4:
            assert slot["pending"] is None
            lo, hi = slot["overlap"]
            v, s = CP.project(x[lo:hi + 1], wkv, wg, ape, np.arange(lo, hi + 1), ratio)
            kv[:4], sc[:4] = v, s                       # the previous-block slots
        else:
            lo, hi = slot["pending"]
            v, s = CP.project(x[lo:hi + 1], wkv, wg, ape, np.arange(lo, hi + 1), ratio)
            kv[lo % ratio:hi % ratio + 1], sc[lo % ratio:hi % ratio + 1] = v, s
        a, _ = CP.compress_stream(x[T:], T, *args, state=full)
        b, _ = CP.compress_stream(x[T:], T, *args, state=(kv, sc))
        assert sorted(a) == sorted(b) and len(a) == (T + more) // ratio - T // ratio
        for i in a:
            np.testing.assert_allclose(a[i], b[i], rtol=1e-12, atol=1e-12)
        # and the slot is not larger than needed: dropping its first token
        # changes the next entry
        kv2, sc2 = kv.copy(), sc.copy()
        first = (0 if ratio == 4 else lo % ratio)
        kv2[first], sc2[first] = 0.0, -np.inf
        c, _ = CP.compress_stream(x[T:], T, *args, state=(kv2, sc2))
        i0 = min(a)
        assert np.abs(c[i0] - a[i0]).max() > 1e-6


def test_scatter_gather_identity():
    rng = np.random.default_rng(5)
    for bs in (32, 1, 4):
        counts = [int(rng.integers(0, 200)) for _ in range(5)]
        nb_total = sum(-(-c // bs) for c in counts) + 7
        table = P.allocate(counts, bs, nb_total, rng)
        for b, n in enumerate(counts):
            E = rng.standard_normal((n, 6))
            pool = P.scatter(E, table[b], bs, nb_total)
            past = -(-n // bs) * bs                   # first entry of the first absent block
            ids = np.concatenate([rng.permutation(n), [-1, past]]).astype(np.int64)
            rows, valid = P.gather(pool, table[b], bs, ids)
            assert np.array_equal(valid, np.concatenate([np.ones(n, bool), [False, False]]))
            np.testing.assert_array_equal(rows[:n], E[ids[:n]])
        # every allocated block belongs to one sequence only
        used = table[table >= 0]
        assert len(np.unique(used)) == len(used)
        # an id past the table or in an unallocated block is absent
        assert P.entry_address(table[0], bs, 10 ** 6) is None
