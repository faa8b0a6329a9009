"""The CSA2 decoder layer group at m = 1 (V4.1-Flash diagram page: CSA2 with
MXFP4 main KV, FP4 index keys, Top-512, and layers that reuse a Full layer's
main KV and top-512 ids), at the shape bench.py runs: batch 8, 262,144
entries (one per token), one Full layer and 5 Reuse layers.  One decode step,
then for the first and last sequence: the entries and index keys the m = 1
compressor wrote, the bf16 index scores and the selection, and the attention
output of every layer of the group, all against the oracle."""

import gc

import numpy as np
import pytest
import torch

from gpu_util import close_bf16, need_gpu, say, score_bound, step_bound, to_np
from kv_cache_decode_csa_amd import _lib, decode, synth
from oracle import attention, codec, indexer, rope
from oracle import topk as TK
from test_gpu_fullsize import check_entry, oracle_new_entries, rows_of

pytestmark = pytest.mark.gpu


def test_csa2_m1_layer_group():
    need_gpu()
    w = synth.WORKLOADS[6]
    R = w.extra["reuse"]
    say(f"full-size step {w.name}: B={w.B} ctx={w.ctx} entries={w.n_entries} reuse={R}")
    layer = decode.CsaDecodeLayer(w, copies=1)
    layer.step()
    torch.cuda.synchronize()
    om = rope.frequencies(w.theta, rope.V4_YARN)
    t, N, B = w.t, w.n_entries, w.B
    ent_dev, keys_dev = layer.sets[0]
    sc = torch.empty((B, 1, N), dtype=torch.float32, device="cuda")
    ids2 = torch.empty_like(layer.topk)
    _lib.csa_index_topk_bf16(*layer.qi_arg, layer.wi, keys_dev, w.key_fmt, layer.pos, 1, B, 1,
                             w.Hi, N, w.topk, ids2, sc, layer.ws_idx)
    torch.cuda.synchronize()
    ids = layer.topk.cpu().numpy()[:, 0]
    assert np.array_equal(ids2.cpu().numpy()[:, 0], ids), "selection differs between calls"
    S16 = sc.cpu().numpy()[:, 0]
    qdev = layer.qi.float().cpu().numpy()[:, 0]
    outs = [to_np(layer.out)[:, 0]] + [to_np(r[3])[:, 0] for r in layer.reuse]
    nv = int(indexer.n_visible(t, 1, N))
    assert nv == N
    new_i = list(range(t - 7, t + 1))  # m = 1: every token of the set-up and the step
    for b in (0, B - 1):
        # 1. entries and index keys written by the m = 1 compressor (no slot bias)
        ref_main = oracle_new_entries(w, b, 512, False, om)
        ref_key = oracle_new_entries(w, b, 128, True, om)
        assert sorted(ref_main) == new_i
        main_rows = rows_of(ent_dev[b, new_i[0]:new_i[-1] + 1], w.ent_fmt, 512)
        key_rows = rows_of(keys_dev[b, new_i[0]:new_i[-1] + 1], w.key_fmt, 128)
        for j, i in enumerate(new_i):
            check_entry(main_rows[j], ref_main[i], w.ent_fmt, 512)
            check_entry(key_rows[j], ref_key[i], w.key_fmt, 128)
        # 2. bf16 scores over every entry and the selection
        qraw, wi = synth.index_queries(w, [b])
        qv = codec.store(qraw[0], "fp4_mx32")[1]
        assert np.array_equal(qdev[b], qv), "index queries are not the oracle's MXFP4 values"
        kval = codec.store(synth.index_keys(w, [b])[0], w.key_fmt)[1]
        for i in new_i:
            kval[i] = codec.store(ref_key[i], w.key_fmt)[1]
        wv = wi[0].astype(np.float64)
        S_ref = indexer.scores(qv, wv, kval, nv)
        tol = score_bound(qv, wv, kval[:nv])
        kstep = np.zeros_like(kval[:nv])
        for i in new_i:  # the compressor's keys may differ by one FP4 step near a tie
            kstep[i] = step_bound(ref_key[i], w.key_fmt, 128)
        tol = tol + (kstep @ np.abs(qv).T) @ np.abs(wv)
        err = np.abs(S16[b, :nv] - S_ref)
        assert np.all(err <= tol + np.abs(S_ref) * 2.0 ** -8 + 1e-30), (b, err.max())
        assert np.array_equal(ids[b], TK.topk(S16[b, :nv], w.topk, nv)), b
        del kval, kstep
        # 3. attention of the Full layer and of every Reuse layer over the ids
        E = synth.entries(w, [b])[0]
        sel = ids[b]
        rows = codec.store(E[np.maximum(sel, 0)], w.ent_fmt)[1]
        for i in new_i:
            rows[sel == i] = codec.store(ref_main[i], w.ent_fmt)[1]
        slots = np.where(sel >= 0, np.arange(len(sel)), -1)
        wid = attention.window_ids(t)
        q, sink = synth.queries(w, [b])
        inputs = [(q[0], sink, synth.window_rows(w, [b])[0])]
        for lay in range(1, R + 1):
            rq, rs, rw = synth.reuse_layer_inputs(w, lay, [b])
            inputs.append((rq[0], rs, rw[0]))
        for lay, (ql, sl, wl) in enumerate(inputs):
            win = codec.store(wl, w.win_fmt)[1]
            ref = attention.sparse_decode(ql.astype(np.float64), win, wid, rows, slots, sl,
                                          512 ** -0.5, t, om)
            close_bf16(outs[lay][b], ref)
        say(f"  b={b}: m=1 entries, FP4 scores and selection, {1 + R} layers' attention ok")
        del E
        gc.collect()
    del layer
    gc.collect()
    torch.cuda.empty_cache()
