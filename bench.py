"""Decode-step benchmark: one MI355X, one CSA (or HCA) layer, synthetic data.

Default workload: CSA decode at 1M context with a quantized cache -- batch 8,
262,144 compressed entries per sequence stored FP8-MX32 (528 B rows), FP8
index keys (132 B), 64 query heads x 512, 64 indexer heads x 128, top-512,
128-row FP8 window.  One step = compress the new token (main KV and index
keys, one csa_compress_many call), score every visible index key and select
the top 512, then attend over the window plus the selection.  All inputs are
resident in HBM before timing.

Prints one JSON line.  value = tokens/s per layer = B / step time.  The
roofline object is for the dominant phase, csa_index_topk (its algorithmic
bytes are the visible index keys plus q_idx, w and the output ids), timed with
HIP events on the stream it runs on.  cpu_baseline times the float64 oracle
(test infrastructure) on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload csa_1m_fp8|csa_1m_mxfp4|
                  csa_1m_fp4idx|csa_1m_fp8_layer|csa_1m_fp8_paged|csa2_m1_256k|
                  csa_64k_bf16|csa_64k_bf16_b128|hca_1m_bf16|hca_1m_bf16_paged|
                  csa_prefill_32k_bf16] [--copies C] [--no-cpu-baseline]

csa_64k_bf16_b128 is the 64K workload at batch 128, where the decode attention
takes one work-group per whole list instead of 64-row chunks and a merge (the
same bits either way).

The *_paged workloads run the same step from a block cache: entries and index
keys in pools of blocks (32 CSA entries or 1 HCA entry per block) found
through per-sequence block tables, windows and compressor slots in a pool of
state slots.

The chunked-prefill workload (32,768 new tokens on a 262,144-token prefix,
batch 1) reports prefill tokens/s per layer; its roofline object is the
indexer's MFMA rate (bf16 TFLOP/s of the heads x 128 x visible-keys
contraction) during csa_index_topk.
  python bench.py --copy-calibration     # known-size copy for HBM byte counters
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {"csa_1m_fp8": 5, "csa_1m_mxfp4": 5, "csa_1m_fp4idx": 5, "csa_1m_fp8_layer": 5,
             "csa_1m_fp8_paged": 5, "csa2_m1_256k": 6, "csa_64k_bf16": 2, "csa_64k_bf16_b128": 2,
             "hca_1m_bf16": 3, "hca_1m_bf16_paged": 3, "csa_prefill_32k_bf16": 4}


# the default workload's metric; the others name what they measure
METRICS = {
    "csa_1m_fp8": "CSA top-512 decode tokens/s per layer at 1M ctx; achieved HBM GB/s vs peak",
    "csa_64k_bf16": "CSA top-512 decode tokens/s per layer at 64K ctx (bf16 cache); achieved HBM "
                    "GB/s vs peak",
    "csa_64k_bf16_b128": "CSA top-512 decode tokens/s per layer at 64K ctx (bf16 cache), batch "
                         "128; achieved HBM GB/s vs peak",
    "hca_1m_bf16": "HCA decode tokens/s per layer at 1M ctx (bf16 cache); achieved HBM GB/s vs "
                   "peak",
    "csa_1m_fp8_layer": "CSA top-512 decode tokens/s per layer at 1M ctx, whole layer (query path, "
                        "window write and output projection included); achieved HBM GB/s vs peak",
    "csa2_m1_256k": "CSA2 m=1 layer-group decode tokens/s per layer at 256K ctx (6 layers sharing "
                    "main KV and top-512 ids); achieved HBM GB/s vs peak",
    "csa_1m_fp8_paged": "CSA top-512 decode tokens/s per layer at 1M ctx from a block cache (32 "
                        "entries per block, state slots); achieved HBM GB/s vs peak",
    "hca_1m_bf16_paged": "HCA decode tokens/s per layer at 1M ctx (bf16 cache) from a block cache "
                         "(1 entry per block, state slots); achieved HBM GB/s vs peak",
}


def row_bytes(fmt, dim):
    return {"f32": 4 * dim, "bf16": 2 * dim, "fp8_mx32": dim + dim // 32,
            "fp4_e4m3_16": dim // 2 + dim // 16, "fp4_mx32": dim // 2 + dim // 32}[fmt]


def algorithmic_bytes(w):
    """Bytes the method must move per step (whole batch), by phase."""
    B, N = w.B, w.n_entries
    qb = 2 if w.q_fmt == "bf16" else 4
    out = {}
    # compressors: weights once per step, x, slot states read+written, one emitted row
    dim = w.dim
    coff = 2 if w.ratio == 4 else 1
    comp_main = (2 * coff * 512 * dim * qb + B * dim * qb
                 + 2 * 2 * B * coff * w.ratio * coff * 512 * 4 + B * row_bytes(w.ent_fmt, 512))
    out["csa_compress"] = comp_main
    if w.ratio != 128:  # CSA: the index-key compressor runs in the same call
        out["csa_compress"] += (2 * coff * 128 * dim * qb + B * dim * qb
                                + 2 * 2 * B * coff * w.ratio * coff * 128 * 4
                                + B * row_bytes(w.key_fmt, 128))
        n_vis = min((w.t + 1) // w.ratio, N)
        # q_idx: bf16, or MXFP4 rows for the FP4 indexer (as the decode layer passes them)
        q_idx = (row_bytes("fp4_mx32", 128) if w.key_fmt == "fp4_mx32" and not w.extra.get("layer")
                 else 128 * qb)
        out["csa_index_topk"] = B * (n_vis * row_bytes(w.key_fmt, 128) + w.Hi * q_idx
                                     + w.Hi * 4 + w.topk * 4)
        k = min(w.topk, n_vis)
        out["csa_sparse_attn_decode"] = B * (k * row_bytes(w.ent_fmt, 512) + k * 4
                                             + 128 * row_bytes(w.win_fmt, 512)
                                             + 2 * w.H * 512 * qb) + w.H * 4
        if w.extra.get("reuse"):  # the layer group: shared rows and ids once, per-layer
            L = 1 + w.extra["reuse"]  # window, q, output and sinks
            out["csa_sparse_attn_group"] = (B * (k * row_bytes(w.ent_fmt, 512) + k * 4)
                                            + L * B * (128 * row_bytes(w.win_fmt, 512)
                                                       + 2 * w.H * 512 * qb) + L * w.H * 4)
            del out["csa_sparse_attn_decode"]
        cfg = w.extra.get("layer")
        if cfg:  # weights once, the token's inputs and outputs (intermediates excluded)
            qr, g, r = cfg["q_rank"], cfg["groups"], cfg["o_rank"]
            wts = dim * qr + qr * w.H * 512 + dim * 512 + qr * w.Hi * 128 + dim * w.Hi
            out["csa_layer_input"] = (2 * wts + 4 * (qr + 512) + B * dim * 2
                                      + B * (w.H * 512 * 2 + w.Hi * 128 * 2 + w.Hi * 4)
                                      + B * row_bytes(w.win_fmt, 512))
            out["csa_layer_output"] = (2 * (r * w.H * 512 + dim * g * r)
                                       + B * w.H * 512 * 2 + B * dim * 2)
    else:
        n_vis = min((w.t + 1) // w.ratio, N)
        out["hca_attn_decode"] = B * (n_vis * row_bytes(w.ent_fmt, 512)
                                      + 128 * row_bytes(w.win_fmt, 512)
                                      + 2 * w.H * 512 * qb) + w.H * 4
    pg = w.extra.get("paged")
    if pg:  # block ids read through the tables (4 B each) and the slot map
        bs = pg["block_entries"]
        n_vis = min((w.t + 1) // w.ratio, N)
        if w.ratio != 128:
            out["csa_index_topk"] += B * (-(-n_vis // bs)) * 4
            out["csa_sparse_attn_decode"] += B * (min(w.topk, n_vis) * 4 + 4)
        else:
            out["hca_attn_decode"] += B * (-(-n_vis // bs) * 4 + 4)
    return out


def prefill_flops(w):
    """Dense-contraction FLOPs of one prefill chunk, by phase (2 per MAC).
    Indexer: every query scores its visible keys with Hi heads x 128 dims.
    Attention: 64 heads x (q.c and p.c over 512 dims) per list row (window +
    top-k).  Compressors: x times both projections of both compressors."""
    from kv_cache_decode_csa_amd import synth
    P, T, N0, N = synth.prefill_shape(w)
    vis = sum(min((P + i + 1) // w.ratio, N) for i in range(T))
    return {"csa_compress": 2.0 * T * w.dim * 2 * (2 * 512 + 2 * 128),
            "csa_index_topk": 2.0 * vis * w.Hi * 128,
            "csa_sparse_attn_decode": 2.0 * 2 * T * w.H * 512 * (128 + w.topk)}


def cpu_baseline_prefill(w, n_q=64, n_tok=1024):
    """The oracle on a bounded sample of the prefill chunk: the bulk
    compressor (both compressors) over n_tok tokens, and n_q sampled queries
    (scoring over every visible key, top-k, gather and attention).  Per-token
    cost = compressor time per token + query time per query; value = 1 / that."""
    from kv_cache_decode_csa_amd import synth
    from oracle import attention, compressor, indexer, rope
    from oracle import topk as TK
    om = rope.frequencies(160000.0, rope.V4_YARN if w.yarn else None)
    threads = os.environ.get("OMP_NUM_THREADS") or str(len(os.sched_getaffinity(0)))
    P, T, N0, N = synth.prefill_shape(w)
    x = synth.prefill_hidden(w, 0, n_tok).astype(np.float64)
    t0 = time.perf_counter()
    for d, idx in ((512, False), (128, True)):
        wkv, wg, ape, norm = synth.compressor_weights(w, d, 4, indexer=idx)
        compressor.compress_bulk(x, P, wkv, wg, ape, norm, om, 4, d, rotate=idx)
    t_comp = (time.perf_counter() - t0) / n_tok
    keys = np.concatenate([synth.prefill_index_keys(w, 0, N0),
                           synth.prefill_index_keys(w, 0, N - N0)]).astype(np.float64)
    ent = synth.prefill_entries(w, 0, N0).astype(np.float64)
    sink = synth.prefill_sink(w)
    rng = np.random.default_rng(5)
    qs = rng.choice(T, n_q, replace=False)
    t_q = 0.0
    for i in qs:
        q = synth.prefill_queries(w, i, i + 1)[0].astype(np.float64)
        qi, wi = synth.prefill_index_queries(w, i, i + 1)
        win = synth.prefill_window(w, i, i + 128).astype(np.float64)
        t0 = time.perf_counter()
        nv = int(indexer.n_visible(P + i, 4, N))
        S = indexer.scores(qi[0].astype(np.float64), wi[0], keys, nv)
        ids = TK.topk(S.astype(np.float32), w.topk, nv)
        rows = ent[np.minimum(np.maximum(ids, 0), N0 - 1)]
        attention.attend(q, np.concatenate([win, rows]),
                         np.concatenate([np.ones(128, bool), ids >= 0]), sink, 512 ** -0.5,
                         P + i, om)
        t_q += time.perf_counter() - t0
    per_tok = t_comp + t_q / n_q
    return {"value": 1.0 / per_tok, "unit": "prefill tokens/s/layer", "cores": int(threads),
            "kind": "oracle",
            "sample": f"bulk compressor (main + index) over {n_tok} of {T} new tokens "
                      f"({t_comp * n_tok:.1f} s) plus {n_q} of {T} queries (scoring over all "
                      f"visible keys, top-k, attention; {t_q:.1f} s) in float64 NumPy, "
                      f"extrapolated per token"}


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "csa_1m_fp8_hbm_traffic.md")


def measured_traffic(workload):
    """HBM bytes per csa_index_topk call from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE runs, copy-calibrated), or None when there is no
    summary for this workload or the kernel sources changed since it was taken."""
    return traffic_with_status(workload)[0]


def traffic_with_status(workload):
    """(bytes or None, status): status says whether the counters were taken on
    the current kernel sources, are stale, or do not exist for this workload."""
    if workload != "csa_1m_fp8" or not os.path.exists(TRAFFIC_PROFILE):
        return None, "no counter run for this workload"
    text = open(TRAFFIC_PROFILE).read()
    m_b = re.search(r"traffic_bytes_per_call: (\d+)", text)
    m_h = re.search(r"sources_sha256: ([0-9a-f]+)", text)
    m_s = re.search(r"sources: (.+)", text)
    if not (m_b and m_h and m_s):
        return None, "counter summary unreadable"
    h = hashlib.sha256()
    for f in m_s.group(1).split():
        path = os.path.join(ROOT, f)
        if not os.path.exists(path):
            return None, f"stale: {f} no longer exists"
        h.update(open(path, "rb").read())
    if h.hexdigest() != m_h.group(1):
        return None, "stale: kernel sources changed since the counters were taken"
    return int(m_b.group(1)), "counters taken on the current kernel sources"


def time_steps(layer, steps, torch):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        layer.step()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def step_percentiles(layer, steps, torch):
    """p10 / p50 / p90 of single-step durations (events around each step)."""
    evs = []
    torch.cuda.synchronize()
    for _ in range(steps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        layer.step()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return {"p10": float(np.percentile(t, 10)), "p50": float(np.percentile(t, 50)),
            "p90": float(np.percentile(t, 90))}


def copy_bandwidth(torch, nbytes=2 << 30, reps=5):
    """Measured device-to-device copy rate (read + write bytes per second):
    the practical streaming ceiling next to the nominal 8 TB/s."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def fp4_recall(layer, w, torch):
    """Mean overlap of the FP4 indexer's top-k (MXFP4 keys and queries, bf16
    scores; the last step's output) with the top-k of float32 scores over the
    unquantized seeded keys and queries, through the library's float32 path."""
    from kv_cache_decode_csa_amd import _lib, synth
    B, N = w.B, w.n_entries
    keys = torch.from_numpy(synth.index_keys(w)).cuda()        # [B, N, 128] f32 values
    qi, wi = synth.index_queries(w)
    qf = torch.from_numpy(qi.astype(np.float32)).cuda().reshape(B, 1, w.Hi, 128)
    wf = torch.from_numpy(wi).cuda().reshape(B, 1, w.Hi)
    ids = torch.empty((B, 1, w.topk), dtype=torch.int32, device="cuda")
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, 1, N, w.topk))
    _lib.csa_index_topk(qf, "f32", wf, keys, "f32", layer.pos, w.ratio, B, 1, w.Hi, N, w.topk, ids,
                        None, ws)
    torch.cuda.synchronize()
    a_ids, b_ids = layer.topk.cpu().numpy()[:, 0], ids.cpu().numpy()[:, 0]
    rec = [len(set(a_ids[b].tolist()) & set(b_ids[b].tolist())) / w.topk for b in range(B)]
    del keys, ws
    torch.cuda.empty_cache()
    return float(np.mean(rec))


def flushed_steps(layer, steps, torch, nbytes=512 << 20):
    """Median single-step time when 512 MB are written between steps (the
    last-level cache then holds none of the step's inputs); the flush itself
    is outside the events."""
    junk = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    evs = []
    torch.cuda.synchronize()
    for i in range(steps):
        junk.fill_(i & 0xff)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        layer.step()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    del junk
    torch.cuda.empty_cache()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def time_phases(layer, steps, torch):
    """Average duration of every phase, each bracketed by events on its stream."""
    acc = {}
    pairs = []
    torch.cuda.synchronize()
    for _ in range(steps):
        for name, fn in layer.phases():
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            pairs.append((name, a, b))
        layer.step_no += 1
    torch.cuda.synchronize()
    for name, a, b in pairs:
        acc.setdefault(name, []).append(a.elapsed_time(b))
    return {k: float(np.mean(v)) for k, v in acc.items()}


def _blas_threads():
    """Threads of the BLAS library NumPy calls (threadpoolctl), else the
    affinity count."""
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except ImportError:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(w, n_seq=None, min_seconds=10.0):
    """The oracle on n_seq sequences of the workload (default: the whole
    batch) for one decode step each: the compressors on the new token (main
    KV and, for CSA, index keys, continuing a state built from the 7 tokens
    before it), decoding the stored index keys, scoring, top-k, decoding the
    selected rows and the window, attention.  Building the stored bytes with
    the oracle's codec and the compressor states is not timed.  The timed part
    is repeated over the same sequences until it has run for at least
    min_seconds; then one sequence's step is timed again with the BLAS pool
    held to a single thread."""
    from kv_cache_decode_csa_amd import synth
    from oracle import attention, codec, compressor, indexer, rope
    from oracle import topk as TK
    n_seq = w.B if n_seq is None else min(n_seq, w.B)
    om = rope.frequencies(160000.0, rope.V4_YARN if w.yarn else None)
    t = w.t
    tail = 7
    comps = [(512, 0, False)] + ([(128, 1, True)] if w.ratio != 128 else [])
    cw = {d: tuple(np.asarray(a, np.float64) for a in synth.compressor_weights(w, d, w.ratio,
                                                                              indexer=ix))
          for d, _, ix in comps}
    prepared = []
    for b in range(n_seq):
        br = [b]
        q, sink = synth.queries(w, br)
        win = synth.window_rows(w, br)[0]
        ent = synth.entries(w, br)[0]
        win_st = codec.store(win, w.win_fmt)[0]
        keys_st = None
        qi = wi = None
        if w.ratio != 128:
            qi, wi = synth.index_queries(w, br)
            keys_st = codec.store(synth.index_keys(w, br)[0], w.key_fmt)[0]
        reuse = [synth.reuse_layer_inputs(w, layer, br)
                 for layer in range(1, w.extra.get("reuse", 0) + 1)]
        reuse = [(rq[0].astype(np.float64), rs, codec.store(rw[0], w.win_fmt)[0])
                 for rq, rs, rw in reuse]
        x = synth.normal_batched(w.seed, synth.T_X, w.B, (1, w.dim), b_range=br)[0]
        xt = synth.normal_batched(w.seed, synth.T_XTAIL, w.B, (tail, w.dim), b_range=br)[0]
        states = {}
        for d, rot, _ in comps:
            wkv, wg, ape, nw = cw[d]
            _, states[d] = compressor.compress_stream(
                np.asarray(xt, np.float64), t - tail, wkv, wg, ape, nw, om, w.ratio, d,
                rotate=bool(rot))
        prepared.append((q, sink, win_st, ent, keys_st, qi, wi, reuse,
                         np.asarray(x, np.float64), states))
    cfg = w.extra.get("layer")
    if cfg:  # the layer's input and output steps are timed too
        from oracle import layer as OL
        lw = {k: v.astype(np.float64) for k, v in synth.layer_weights(
            w.seed, w.dim, cfg["q_rank"], w.H, w.Hi, cfg["groups"], cfg["o_rank"]).items()}
        lw.update(H=w.H, Hi=w.Hi)
        xs = [synth.hidden(w, 1, idx=b)[0].astype(np.float64) for b in range(n_seq)]

    def one(si):
        """One sequence's decode step; returns its timed seconds."""
        q, sink, win_st, ent, keys_st, qi, wi, reuse, x, states = prepared[si]
        dt = 0.0
        t0 = time.perf_counter()
        if cfg:
            OL.layer_input(xs[si], t, lw, om)
        for d, rot, _ in comps:
            wkv, wg, ape, nw = cw[d]
            compressor.compress_stream(x, t, wkv, wg, ape, nw, om, w.ratio, d, rotate=bool(rot),
                                       state=states[d])
        if w.ratio != 128:
            K = codec.load(keys_st, w.key_fmt, 128)
            nv = int(indexer.n_visible(t, w.ratio, w.n_entries))
            S = indexer.scores(qi[0].astype(np.float64), wi[0], K, nv)
            ids = TK.topk(S.astype(np.float32), w.topk, nv)
            dt += time.perf_counter() - t0
            rows_st = codec.store(ent[np.maximum(ids, 0)], w.ent_fmt)[0]  # stored rows read
        else:
            dt += time.perf_counter() - t0
            ids = attention.hca_ids(t, w.ratio, w.n_entries)
            rows_st = codec.store(ent[ids], w.ent_fmt)[0]
        t0 = time.perf_counter()
        E = codec.load(rows_st, w.ent_fmt, 512)
        Wv = codec.load(win_st, w.win_fmt, 512)
        wid = attention.window_ids(t)
        rows = np.concatenate([Wv[np.maximum(wid, 0)], E])
        valid = np.concatenate([wid >= 0, ids >= 0])
        o = attention.attend(q[0].astype(np.float64), rows, valid, sink, 512 ** -0.5, t, om)
        if cfg:
            OL.output_projection(o, lw["wo_a"], lw["wo_b"])
        for rq, rs, rw_st in reuse:  # reuse layers: their own q and window
            Rv = codec.load(rw_st, w.win_fmt, 512)
            rows = np.concatenate([Rv[np.maximum(wid, 0)], E])
            attention.attend(rq, rows, valid, rs, 512 ** -0.5, t, om)
        return dt + time.perf_counter() - t0

    threads = _blas_threads()
    t_total, passes = 0.0, 0
    while t_total < min_seconds and passes < 50:
        passes += 1
        for si in range(n_seq):
            t_total += one(si)
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            single = one(0)
    except ImportError:
        pass
    layers = 1 + len(prepared[0][7])
    n_tok = passes * n_seq * layers
    timed = ("compressors (main KV" + (" and index keys" if w.ratio != 128 else "") + "), "
             + ("layer input steps, " if cfg else "")
             + ("key decode, scoring, top-k, " if w.ratio != 128 else "")
             + "row decode and attention" + (", output projection" if cfg else ""))
    scope = ("the whole batch" if n_seq == w.B else f"{n_seq} of {w.B} sequences")
    return {"value": n_tok / t_total, "unit": "tokens/s/layer", "cores": int(threads),
            "kind": "oracle",
            "blas_threads": int(threads),
            "seconds_per_step_whole_batch": t_total / passes * (w.B / n_seq),
            "single_thread_seconds_one_sequence": single,
            "sample": f"{scope} of the same workload at full context ({w.n_entries} entries "
                      f"each), {passes} passes ({n_tok} layer-token steps); timed: {timed} in "
                      f"float64 NumPy with {threads} BLAS threads, {t_total:.1f} s; then one "
                      f"sequence's step on one thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="csa_1m_fp8", choices=sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=None,
                    help="independent cache copies rotated per step (default: at least 4 and "
                         "at least 1 GB of step reads in all, so that no step finds the cache "
                         "lines of an earlier step in the 256 MB last-level cache)")
    ap.add_argument("--cpu-seqs", type=int, default=None,
                    help="sequences the oracle baseline times (default: the whole batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the flushed-cache steps (kernel-trace runs: their averages then "
                         "cover only the steady-state steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the known-size "
                         "reference for HBM byte counters) and exit")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(one process drives one GPU); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if a.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return
    from kv_cache_decode_csa_amd import decode, synth

    w = synth.WORKLOADS[WORKLOADS[a.workload]]
    if a.workload == "csa_prefill_32k_bf16":
        return main_prefill(a, w, torch)
    if a.workload == "csa_1m_mxfp4":
        w = synth.mxfp4_variant(w)
    if a.workload == "csa_1m_fp4idx":
        w = synth.fp4_indexer_variant(w)
    if a.workload == "csa_1m_fp8_layer":
        w = synth.layer_variant(w)
    if a.workload.endswith("_paged"):
        w = synth.paged_variant(w)
    if a.workload == "csa_64k_bf16_b128":
        w = synth.batch_variant(w, 128)
    print(f"# building {a.workload}: B={w.B} ctx={w.ctx} entries={w.n_entries}", file=sys.stderr,
          flush=True)
    t0 = time.time()
    Layer = decode.CsaDecodeLayer if w.ratio != 128 else decode.HcaDecodeLayer
    if a.copies is None:
        step_bytes = sum(algorithmic_bytes(w).values())
        a.copies = max(4, -(-1_000_000_000 // step_bytes))
    layer = Layer(w, copies=a.copies)
    torch.cuda.synchronize()
    print(f"# inputs resident in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    for _ in range(a.warmup):
        layer.step()
    ms = time_steps(layer, a.steps, torch)
    phases = time_phases(layer, a.steps, torch)
    pct = step_percentiles(layer, a.steps, torch)
    flushed_ms = None if a.no_flush else flushed_steps(layer, a.steps, torch)
    copy_gbs = copy_bandwidth(torch)
    ab = algorithmic_bytes(w)
    dom = "csa_index_topk" if w.ratio != 128 else "hca_attn_decode"
    layers = 1 + w.extra.get("reuse", 0)  # layers per step (a layer group with reuse)
    dom_gbs = ab[dom] / (phases[dom] * 1e-3) / 1e9
    traffic, traffic_status = traffic_with_status(a.workload)
    step_bytes = sum(ab.values())
    res = {
        "metric": METRICS.get(w.name, METRICS["csa_1m_fp8"]),
        "value": layers * w.B / (ms * 1e-3),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "context": w.ctx, "entries": w.n_entries,
                   "heads": w.H, "index_heads": w.Hi, "topk": w.topk, "ratio": w.ratio,
                   "kv_format": w.ent_fmt, "window_format": w.win_fmt,
                   "index_key_format": w.key_fmt, "cache_copies": a.copies,
                   "layers_per_step": layers},
        "roofline": {"bound": "hbm", "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dom_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_status": traffic_status, "kernel": dom,
                     "bytes_per_launch": ab[dom], "ms_per_launch": phases[dom]},
        "step_hbm_GBps": step_bytes / (ms * 1e-3) / 1e9,
        "step_ms_percentiles": pct,
        "flushed_step_ms_p50": flushed_ms,
        "measured_copy_GBps": copy_gbs,
        "frac_of_measured_copy": dom_gbs / copy_gbs,
        "phases_ms": phases,
        "algorithmic_bytes": ab,
    }
    if w.key_fmt == "fp4_mx32":
        res["fp4_indexer_recall_vs_f32"] = fp4_recall(layer, w, torch)
    if not a.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_seqs)
    print(json.dumps(res), flush=True)


def main_prefill(a, w, torch):
    from kv_cache_decode_csa_amd import prefill, synth
    P, T, N0, N = synth.prefill_shape(w)
    print(f"# building {a.workload}: {T} new tokens on a {P}-token prefix", file=sys.stderr,
          flush=True)
    t0 = time.time()
    layer = prefill.CsaPrefillChunk(w)
    torch.cuda.synchronize()
    print(f"# inputs resident in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        layer.step()
    ms = time_steps(layer, a.steps, torch)
    phases = time_phases(layer, a.steps, torch)
    pct = step_percentiles(layer, a.steps, torch)
    fl = prefill_flops(w)
    dom = "csa_index_topk"
    tf = fl[dom] / (phases[dom] * 1e-3) / 1e12
    res = {
        "metric": "CSA chunked-prefill tokens/s per layer (32K new tokens on a 256K prefix); "
                  "indexer MFMA TFLOP/s vs peak",
        "value": T / (ms * 1e-3),
        "unit": "prefill tokens/s/layer",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": 1, "prefix": P, "new_tokens": T,
                   "entries_after": N, "heads": w.H, "index_heads": w.Hi, "topk": w.topk,
                   "ratio": w.ratio, "kv_format": "bf16", "window": "linear"},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": dom, "flops_per_launch": fl[dom], "ms_per_launch": phases[dom]},
        "phases_ms": phases,
        "step_ms_percentiles": pct,
        "phase_tflops": {k: fl[k] / (phases[k] * 1e-3) / 1e12 for k in fl},
        "flops": fl,
    }
    if not a.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_prefill(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
