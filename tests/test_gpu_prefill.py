"""Full-size chunked-prefill parity (GPU), in the launch configuration that
bench.py times for the prefill workload: 32,768 new tokens (hidden size 4096)
on a 262,144-token prefix whose 65,536 compressed entries and index keys are
seeded N(0,1) bf16 rows; 64 heads, 64 indexer heads, top-512, a linear raw
window.  One step runs both compressors over the chunk, scores and selects for
every query with causal visibility, and attends.  The oracle starts from the
seeded values (never from the library's bytes) and checks:

* sampled entries and index keys the chunk emitted, within one bf16 step;
* the index scores of sampled queries over every visible key (prefix keys
  exact inputs; emitted keys within their bf16 step, which widens the bound),
  and their selection (a valid top-k of the library's scores that equals the
  oracle's away from near-ties);
* the attention output of the sampled queries over the library's own index
  set, within the bf16 tolerance.
"""

import gc

import numpy as np
import pytest
import torch

from kv_cache_decode_csa_amd import _lib, prefill, synth
from oracle import attention, compressor, indexer, rope

from gpu_util import check_selection, close_bf16, need_gpu, say, score_bound, step_bound, to_np

pytestmark = pytest.mark.gpu


def oracle_chunk_entries(w, d, indexer_side, om):
    """Entries the chunk emits, from the prefix's last block and the chunk's tokens."""
    P, T, N0, N = synth.prefill_shape(w)
    wkv, wg, ape, norm = synth.compressor_weights(w, d, 4, indexer=indexer_side)
    tail = synth.prefill_tail(w).astype(np.float64)
    _, state = compressor.compress_stream(tail, P - 4, wkv, wg, ape, norm, om, 4, d,
                                          rotate=indexer_side)
    x = synth.prefill_hidden(w, 0, T).astype(np.float64)
    out, _ = compressor.compress_bulk(x, P, wkv, wg, ape, norm, om, 4, d, rotate=indexer_side,
                                      state=state)
    del x
    return np.stack([out[i] for i in range(N0, N)])


def bf16_rows(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_prefill_chunk_fullsize():
    need_gpu()
    w = synth.WORKLOADS[4]
    P, T, N0, N = synth.prefill_shape(w)
    say(f"full-size prefill {w.name}: {T} new tokens on {P}, entries {N0} -> {N}")
    layer = prefill.CsaPrefillChunk(w)
    layer.step()
    torch.cuda.synchronize()
    ids = layer.topk.cpu().numpy()[0]                     # [T, k]
    # scores through the library's own output buffer, same inputs as the step
    sc = torch.empty((1, T, N), dtype=torch.float32, device="cuda")
    ids2 = torch.empty_like(layer.topk)
    _lib.csa_index_topk(layer.qi, "bf16", layer.wi, layer.keys, "bf16", layer.pos, 4, 1, T,
                        w.Hi, N, w.topk, ids2, sc, layer.ws_idx)
    torch.cuda.synchronize()
    assert np.array_equal(ids2.cpu().numpy()[0], ids), "selection differs between calls"
    del ids2

    rng = np.random.default_rng(4)
    qs = sorted(set([0, 1, 2, 3, T - 4, T - 3, T - 2, T - 1]
                    + rng.choice(T, 8, replace=False).tolist()))
    S_gpu = sc[0, qs].cpu().numpy()
    del sc
    gc.collect()
    torch.cuda.empty_cache()
    out = to_np(layer.out[0, qs])                         # [n, H, 512]

    om = rope.frequencies(w.theta, rope.V4_YARN)
    # 1. emitted rows
    ref_keys = oracle_chunk_entries(w, 128, True, om)     # [N - N0, 128] float64
    ref_main = oracle_chunk_entries(w, 512, False, om)    # [N - N0, 512]
    samp = np.unique(np.concatenate([[0, N - N0 - 1], rng.choice(N - N0, 62, replace=False)]))
    got_k = bf16_rows(layer.keys[0, N0 + samp])
    got_m = bf16_rows(layer.ent[0, N0 + samp])
    for j, i in enumerate(samp):
        for got, ref, d in ((got_k[j], ref_keys[i], 128), (got_m[j], ref_main[i], 512)):
            err = np.abs(got - ref)
            assert np.all(err <= step_bound(ref, "bf16", d)), (i, d, err.max())
    say(f"  {len(samp)} emitted entries and index keys ok")
    # the prefix rows are stored exactly
    rs = rng.choice(N0, 64, replace=False)
    assert np.array_equal(bf16_rows(layer.keys[0, rs]),
                          np.stack([synth.prefill_index_keys(w, r, r + 1)[0] for r in rs]))

    # 2. scores and selection; the oracle's keys are its own stored values
    keys = np.concatenate([synth.prefill_index_keys(w, 0, N0).astype(np.float64),
                           synth.bf16_round(ref_keys.astype(np.float32)).astype(np.float64)])
    kstep = np.zeros_like(keys)
    kstep[N0:] = step_bound(ref_keys, "bf16", 128)        # an emitted key may differ by this
    ent = synth.prefill_entries(w, 0, N0)
    sink = synth.prefill_sink(w)
    for n, i in enumerate(qs):
        t = P + i
        qi, wi = synth.prefill_index_queries(w, i, i + 1)
        qi, wi = qi[0].astype(np.float64), wi[0].astype(np.float64)
        nv = int(indexer.n_visible(t, 4, N))
        S_ref = indexer.scores(qi, wi, keys, nv)
        tol = score_bound(qi, wi, keys[:nv]) + (kstep[:nv] @ np.abs(qi).T) @ np.abs(wi)
        err = np.abs(S_gpu[n, :nv] - S_ref)
        assert np.all(err <= tol), (i, err.max())
        check_selection(ids[i], S_gpu[n], S_ref, tol, nv, w.topk)
        # 3. attention over the library's own index set
        sel = ids[i]
        rows = np.zeros((len(sel), 512))
        old = (sel >= 0) & (sel < N0)
        rows[old] = ent[sel[old]]
        new = sel >= N0
        rows[new] = synth.bf16_round(ref_main[sel[new] - N0].astype(np.float32))
        # window rows i .. i+127 hold positions t-127 .. t (linear: row = pos - (P-127))
        win = synth.prefill_window(w, i, i + 128)
        wid = attention.window_ids(t, mode="linear", base=P - 127, n_rows=T + 127) - i
        q = synth.prefill_queries(w, i, i + 1)[0].astype(np.float64)
        slots = np.where(sel >= 0, np.arange(len(sel)), -1)
        ref = attention.sparse_decode(q, win.astype(np.float64), wid, rows, slots, sink,
                                      512 ** -0.5, t, om)
        close_bf16(out[n], ref)
        say(f"  query {i}: {nv} visible, scores (max err {err.max():.2e}), selection and "
            f"attention ok")
    del layer
    gc.collect()
    torch.cuda.empty_cache()
