"""The block cache at the bench's full sizes (GPU): one decode step of the
1M-context CSA workload (B 8, 262,144 FP8 entries and keys per sequence) and
of the 1M-context HCA workload (B 16, 8,192 bf16 entries per sequence), each
built twice from the same seeded inputs -- contiguous, and served from a block
cache with shuffled blocks and state slots, as bench.py's *_paged workloads
run it.  The paged step must reproduce the contiguous step bit for bit: the
selected ids, the attention output, the emitted entries and index keys (read
back through the block table) and the compressor slot states.  The
contiguous step itself is checked against the oracle by the other full-size
tests."""

import gc

import pytest
import torch

from kv_cache_decode_csa_amd import decode, synth

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _entry_rows(pool, cache, b, ids):
    """Rows of logical entries ids of sequence b from a block pool."""
    out = []
    for i in ids:
        blk = int(cache.table[b, i // cache.bs])
        out.append(pool[blk, i % cache.bs])
    return torch.stack(out)


def test_csa_1m_paged_step_equals_contiguous():
    need_gpu()
    w = synth.WORKLOADS[5]
    say(f"paged full size {w.name}: B={w.B} entries={w.n_entries}")
    ref = decode.CsaDecodeLayer(w, copies=1)
    ref.step()
    torch.cuda.synchronize()
    ids_ref, out_ref = ref.topk.clone(), ref.out.clone()
    ent_ref, keys_ref = ref.sets[0]
    new = [w.t // 4 - 1, w.t // 4]              # from the hidden tail, and this step's
    rows_ref = [(ent_ref[:, new].clone(), keys_ref[:, new].clone())]
    st_ref = [(c.kv.clone(), c.sc.clone()) for c in ref.comp[0]]
    del ref
    _free()
    pg = decode.CsaDecodeLayer(synth.paged_variant(w), copies=1)
    pg.step()
    torch.cuda.synchronize()
    assert torch.equal(pg.topk, ids_ref)
    assert torch.equal(pg.out.view(torch.int16), out_ref.view(torch.int16))
    ent, keys = pg.sets[0]
    c = pg.cache
    for b in range(w.B):
        assert torch.equal(_entry_rows(ent, c, b, new), rows_ref[0][0][b])
        assert torch.equal(_entry_rows(keys, c, b, new), rows_ref[0][1][b])
    for comp, (kv, sc) in zip(pg.comp[0], st_ref):
        s = c.slot.long()
        assert torch.equal(comp.kv[s], kv) and torch.equal(comp.sc[s], sc)
    say("  ids, output, emitted rows and slot states equal")
    del pg
    _free()


def test_hca_1m_paged_step_equals_contiguous():
    need_gpu()
    w = synth.WORKLOADS[3]
    say(f"paged full size {w.name}: B={w.B} entries={w.n_entries}")
    ref = decode.HcaDecodeLayer(w, copies=1)
    ref.step()
    torch.cuda.synchronize()
    out_ref = ref.out.clone()
    st_ref = (ref.comp[0].kv.clone(), ref.comp[0].sc.clone())
    del ref
    _free()
    pg = decode.HcaDecodeLayer(synth.paged_variant(w), copies=1)
    pg.step()
    torch.cuda.synchronize()
    assert torch.equal(pg.out.view(torch.int16), out_ref.view(torch.int16))
    s = pg.cache.slot.long()
    assert torch.equal(pg.comp[0].kv[s], st_ref[0]) and torch.equal(pg.comp[0].sc[s], st_ref[1])
    say("  output and slot states equal")
    del pg
    _free()
