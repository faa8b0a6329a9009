"""Sparse (CSA) and dense (HCA) attention parity against the oracle (GPU).

The index lists are generated inputs (distinct ids, -1 padding, duplicates,
ids outside the entry buffer), so attention is checked on its own; the fused
path is covered by the whole-path tests.  bf16 outputs: |g - r| <= 1e-2 +
2e-2 |r|; float32 path: 1e-5.
"""

import numpy as np
import pytest
import torch

from kv_cache_decode_csa_amd import _lib, synth
from oracle import attention as A
from oracle import codec, rope

from gpu_util import (bf16, close_bf16, close_f32, f32, i32, need_gpu, rope_tables, say, to_np,
                      upload_rows)

pytestmark = pytest.mark.gpu
OM = rope.frequencies(160000.0, rope.V4_YARN)
ROPE_ROWS = 1 << 20


@pytest.fixture(scope="module")
def tables():
    need_gpu()
    return rope_tables(ROPE_ROWS)


def gen_ids(rng, n_vis, k, n_max):
    """k ids: mostly distinct visible ids, plus -1s, a duplicate and an id past Nmax."""
    m = min(k, n_vis)
    ids = rng.choice(n_vis, size=m, replace=False).astype(np.int32) if m else np.zeros(0, np.int32)
    ids = np.concatenate([ids, np.full(k - m, -1, np.int32)])
    if k >= 8 and m >= 4:
        ids[1] = ids[0]          # duplicate row
        ids[3] = -1
        ids[5] = n_max + 7       # outside the buffer: absent
    return ids


def oracle_sparse(qv, winv, entv, ids, sink, pos, mode="ring", base=0, n_rows=128, scale=None):
    scale = 512 ** -0.5 if scale is None else scale
    wid = A.window_ids(pos, mode, base, n_rows=n_rows if mode == "linear" else None)
    ids = np.where((ids >= 0) & (ids < len(entv)), ids, -1)
    return A.sparse_decode(qv, winv, wid, entv, ids, sink, scale, pos, OM)


@pytest.mark.parametrize("efmt,wfmt", [("bf16", "bf16"), ("fp8_mx32", "fp8_mx32"),
                                       ("fp4_e4m3_16", "fp8_mx32"), ("bf16", "fp8_mx32"),
                                       ("mix576", "fp8_mx32"), ("mix576", "bf16")])
@pytest.mark.parametrize("k", [512, 37, 0])
def test_csa_decode(tables, efmt, wfmt, k):
    cos, sin = tables
    B, H, N = 3, 64, 3000
    rng = np.random.default_rng(hash((efmt, wfmt, k)) % 1000)
    q = synth.bf16_round(rng.standard_normal((B, 1, H, 512)).astype(np.float32))
    win = rng.standard_normal((B, 128, 512)).astype(np.float32)
    ent = rng.standard_normal((B, N, 512)).astype(np.float32)
    if efmt == "bf16":
        ent = synth.bf16_round(ent)
    if wfmt == "bf16":
        win = synth.bf16_round(win)
    sink = rng.standard_normal(H).astype(np.float32)
    pos = np.array([[4 * N - 1], [60], [1000]], np.int32)
    ids = np.stack([gen_ids(rng, min((int(pos[b, 0]) + 1) // 4, N), k, N) for b in range(B)])
    ids = ids.reshape(B, 1, k)
    say(f"csa attn {efmt}/{wfmt} k={k}")
    out = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(B, 1, H, k))
    _lib.csa_sparse_attn_decode(bf16(q), "bf16", upload_rows(win, wfmt), wfmt, _lib.WIN_RING128,
                                None, 128, upload_rows(ent, efmt), efmt, N,
                                i32(ids) if k else None, k, i32(pos), B, 1, H, f32(sink),
                                512 ** -0.5, cos, sin, out, "bf16", ws)
    got = to_np(out)
    winv = codec.store(win, wfmt)[1]
    entv = codec.store(ent, efmt)[1]
    for b in range(B):
        ref = oracle_sparse(q[b, 0].astype(np.float64), winv[b], entv[b], ids[b, 0], sink,
                            int(pos[b, 0]))
        close_bf16(got[b, 0], ref)


def test_csa_multi_query_linear_window_and_heads(tables):
    cos, sin = tables
    B, Q, H, N, k = 2, 3, 128, 800, 100
    rng = np.random.default_rng(21)
    q = synth.bf16_round(rng.standard_normal((B, Q, H, 512)).astype(np.float32))
    WR = 300
    win = synth.bf16_round(rng.standard_normal((B, WR, 512)).astype(np.float32))
    ent = rng.standard_normal((B, N, 512)).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    base = np.array([1000, 0], np.int32)
    pos = np.array([[1100, 1299, 1350], [5, 250, 299]], np.int32)  # 1350 > base+WR-1: rows absent
    ids = np.stack([np.stack([gen_ids(rng, min((int(p) + 1) // 4, N), k, N) for p in pos[b]])
                    for b in range(B)])
    out = torch.empty((B, Q, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(B, Q, H, k))
    _lib.csa_sparse_attn_decode(bf16(q), "bf16", bf16(win), "bf16", _lib.WIN_LINEAR, i32(base), WR,
                                upload_rows(ent, "fp8_mx32"), "fp8_mx32", N, i32(ids), k, i32(pos),
                                B, Q, H, f32(sink), 512 ** -0.5, cos, sin, out, "bf16", ws)
    got = to_np(out)
    entv = codec.store(ent, "fp8_mx32")[1]
    for b in range(B):
        for qq in range(Q):
            ref = oracle_sparse(q[b, qq].astype(np.float64), win[b].astype(np.float64), entv[b],
                                ids[b, qq], sink, int(pos[b, qq]), "linear", int(base[b]), WR)
            close_bf16(got[b, qq], ref)


@pytest.mark.parametrize("k,efmt", [(512, "bf16"), (1300, "fp8_mx32"), (45, "fp4_e4m3_16"),
                                    (512, "mix576")])
def test_csa_many_queries_long_chunks(tables, k, efmt):
    """16+ queries per sequence: a work-group takes up to 640 list rows (the
    whole window + top-512 list finishes without partials; longer lists are
    split into 640-row chunks and merged)."""
    cos, sin = tables
    B, Q, H, N = 2, 20, 64, 2500
    rng = np.random.default_rng(1000 + k)
    q = synth.bf16_round(rng.standard_normal((B, Q, H, 512)).astype(np.float32))
    WR = Q + 127
    win = synth.bf16_round(rng.standard_normal((B, WR, 512)).astype(np.float32))
    ent = rng.standard_normal((B, N, 512)).astype(np.float32)
    if efmt == "bf16":
        ent = synth.bf16_round(ent)
    sink = rng.standard_normal(H).astype(np.float32)
    P = np.array([4 * N - Q, 700], np.int32)             # first new position per sequence
    base = P - 127
    pos = P[:, None] + np.arange(Q, dtype=np.int32)[None]
    ids = np.stack([np.stack([gen_ids(rng, min((int(p) + 1) // 4, N), k, N) for p in pos[b]])
                    for b in range(B)])
    say(f"csa attn long chunks k={k} {efmt}")
    out = torch.empty((B, Q, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(B, Q, H, k))
    _lib.csa_sparse_attn_decode(bf16(q), "bf16", bf16(win), "bf16", _lib.WIN_LINEAR, i32(base), WR,
                                upload_rows(ent, efmt), efmt, N, i32(ids), k, i32(pos),
                                B, Q, H, f32(sink), 512 ** -0.5, cos, sin, out, "bf16", ws)
    got = to_np(out)
    entv = codec.store(ent, efmt)[1]
    for b in range(B):
        for qq in range(Q):
            ref = oracle_sparse(q[b, qq].astype(np.float64), win[b].astype(np.float64), entv[b],
                                ids[b, qq], sink, int(pos[b, qq]), "linear", int(base[b]), WR)
            close_bf16(got[b, qq], ref)


@pytest.mark.parametrize("H,k", [(32, 512), (128, 700)])
def test_csa_many_queries_other_head_counts(tables, H, k):
    """16+ queries per sequence with H != 64 take the 16-head-group kernel in
    its long-chunk form (640-row chunks, ids staged in LDS), merged when the
    list spans several chunks."""
    cos, sin = tables
    B, Q, N = 1, 17, 1500
    rng = np.random.default_rng(2000 + H)
    q = synth.bf16_round(rng.standard_normal((B, Q, H, 512)).astype(np.float32))
    WR = Q + 127
    win = synth.bf16_round(rng.standard_normal((B, WR, 512)).astype(np.float32))
    ent = synth.bf16_round(rng.standard_normal((B, N, 512)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    P = np.array([4 * N - Q], np.int32)
    base = P - 127
    pos = P[:, None] + np.arange(Q, dtype=np.int32)[None]
    ids = np.stack([np.stack([gen_ids(rng, min((int(p) + 1) // 4, N), k, N) for p in pos[b]])
                    for b in range(B)])
    say(f"csa attn long chunks H={H} k={k}")
    out = torch.empty((B, Q, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(B, Q, H, k))
    _lib.csa_sparse_attn_decode(bf16(q), "bf16", bf16(win), "bf16", _lib.WIN_LINEAR, i32(base), WR,
                                bf16(ent), "bf16", N, i32(ids), k, i32(pos), B, Q, H, f32(sink),
                                512 ** -0.5, cos, sin, out, "bf16", ws)
    got = to_np(out)
    for qq in range(Q):
        ref = oracle_sparse(q[0, qq].astype(np.float64), win[0].astype(np.float64),
                            ent[0].astype(np.float64), ids[0, qq], sink, int(pos[0, qq]),
                            "linear", int(base[0]), WR)
        close_bf16(got[0, qq], ref)


@pytest.mark.parametrize("efmt,wfmt,k,H,B", [("fp8_mx32", "fp8_mx32", 512, 64, 70),
                                             ("bf16", "bf16", 512, 64, 70),
                                             ("fp4_e4m3_16", "fp8_mx32", 37, 64, 70),
                                             ("mix576", "fp8_mx32", 512, 64, 70),
                                             ("fp8_mx32", "bf16", 200, 128, 34),
                                             ("fp8_mx32", "fp8_mx32", 0, 64, 70)])
def test_batch_invariant_whole_lists(tables, efmt, wfmt, k, H, B):
    """A batch with at least 256 (sequence, 16-head group) items runs one
    work-group per list; a small batch splits each list into 64-row chunks
    and merges them.  Every sequence's output must be the same bits either
    way (the decode output does not depend on the batch), and equal the
    oracle within the bf16 tolerance."""
    cos, sin = tables
    N, sub = 600, 10
    assert _lib.csa_sparse_attn_workspace_size(B, 1, H, k) <= 1   # one work-group per list
    assert _lib.csa_sparse_attn_workspace_size(sub, 1, H, k) > 1  # chunks and partials
    rng = np.random.default_rng(4000 + k + H)
    q = synth.bf16_round(rng.standard_normal((B, 1, H, 512)).astype(np.float32))
    win = rng.standard_normal((B, 128, 512)).astype(np.float32)
    ent = rng.standard_normal((B, N, 512)).astype(np.float32)
    if efmt == "bf16":
        ent = synth.bf16_round(ent)
    if wfmt == "bf16":
        win = synth.bf16_round(win)
    sink = rng.standard_normal(H).astype(np.float32)
    # full lists, padded lists (few visible entries) and partial windows
    pos = rng.integers(4 * N - 8, 4 * N + 5000, size=(B, 1)).astype(np.int32)
    pos[1::7, 0] = rng.integers(100, max(4 * k, 200), size=len(pos[1::7]))
    ids = np.stack([gen_ids(rng, min((int(pos[b, 0]) + 1) // 4, N), k, N)
                    for b in range(B)]).reshape(B, 1, k)
    say(f"batch invariance {efmt}/{wfmt} k={k} H={H}: B={B} against sub-batches of {sub}")
    qd, wd, ed = bf16(q), upload_rows(win, wfmt), upload_rows(ent, efmt)
    idd, pd, sd = i32(ids), i32(pos), f32(sink)

    def run(b0, b1):
        n = b1 - b0
        sl = [t[b0:b1].clone() for t in (qd, wd, ed, idd, pd)]  # fresh, aligned buffers
        out = torch.empty((n, 1, H, 512), dtype=torch.bfloat16, device="cuda")
        ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(n, 1, H, k))
        _lib.csa_sparse_attn_decode(sl[0], "bf16", sl[1], wfmt, _lib.WIN_RING128, None, 128,
                                    sl[2], efmt, N, sl[3], k, sl[4], n, 1, H, sd,
                                    512 ** -0.5, cos, sin, out, "bf16", ws)
        return out

    whole = run(0, B)
    split = torch.cat([run(b0, min(b0 + sub, B)) for b0 in range(0, B, sub)])
    torch.cuda.synchronize()
    same = torch.eq(whole.view(torch.int16), split.view(torch.int16))
    assert bool(same.all()), f"{int((~same).sum())} outputs differ between the two work splits"
    got = to_np(whole)
    winv = codec.store(win[[0, 1, B - 1]], wfmt)[1]
    entv = codec.store(ent[[0, 1, B - 1]], efmt)[1]
    for i, b in enumerate([0, 1, B - 1]):
        ref = oracle_sparse(q[b, 0].astype(np.float64), winv[i], entv[i], ids[b, 0], sink,
                            int(pos[b, 0]))
        close_bf16(got[b, 0], ref)


def test_batch_invariant_whole_lists_multi_query(tables):
    """Three queries per sequence (consecutive positions, as in speculative
    decoding): 22 sequences x 3 queries x 4 head groups take one work-group
    per list, pairs of sequences take 64-row chunks and the merge; the same
    bits either way, and the oracle's values."""
    cos, sin = tables
    B, Q, H, N, k, sub = 22, 3, 64, 700, 300, 2
    rng = np.random.default_rng(4321)
    q = synth.bf16_round(rng.standard_normal((B, Q, H, 512)).astype(np.float32))
    win = rng.standard_normal((B, 128, 512)).astype(np.float32)
    ent = rng.standard_normal((B, N, 512)).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    p0 = rng.integers(130, 4 * N, size=B).astype(np.int32)
    pos = (p0[:, None] + np.arange(Q, dtype=np.int32)[None]).astype(np.int32)
    ids = np.stack([np.stack([gen_ids(rng, min((int(p) + 1) // 4, N), k, N) for p in pos[b]])
                    for b in range(B)])
    assert _lib.csa_sparse_attn_workspace_size(B, Q, H, k) <= 1
    assert _lib.csa_sparse_attn_workspace_size(sub, Q, H, k) > 1
    say(f"batch invariance, {Q} queries per sequence: B={B} against sub-batches of {sub}")
    qd, wd, ed = bf16(q), upload_rows(win, "fp8_mx32"), upload_rows(ent, "fp8_mx32")
    idd, pd, sd = i32(ids), i32(pos), f32(sink)

    def run(b0, b1):
        n = b1 - b0
        sl = [t[b0:b1].clone() for t in (qd, wd, ed, idd, pd)]
        out = torch.empty((n, Q, H, 512), dtype=torch.bfloat16, device="cuda")
        ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(n, Q, H, k))
        _lib.csa_sparse_attn_decode(sl[0], "bf16", sl[1], "fp8_mx32", _lib.WIN_RING128, None, 128,
                                    sl[2], "fp8_mx32", N, sl[3], k, sl[4], n, Q, H, sd,
                                    512 ** -0.5, cos, sin, out, "bf16", ws)
        return out

    whole = run(0, B)
    split = torch.cat([run(b0, min(b0 + sub, B)) for b0 in range(0, B, sub)])
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16), split.view(torch.int16))
    got = to_np(whole)
    winv = codec.store(win[[0, B - 1]], "fp8_mx32")[1]
    entv = codec.store(ent[[0, B - 1]], "fp8_mx32")[1]
    for i, b in enumerate([0, B - 1]):
        for qq in range(Q):
            ref = oracle_sparse(q[b, qq].astype(np.float64), winv[i], entv[i], ids[b, qq], sink,
                                int(pos[b, qq]))
            close_bf16(got[b, qq], ref)


@pytest.mark.parametrize("efmt", ["bf16", "fp8_mx32", "fp4_e4m3_16", "mix576"])
def test_hca_decode(tables, efmt):
    cos, sin = tables
    B, H, N = 3, 64, 2500
    rng = np.random.default_rng(31)
    q = synth.bf16_round(rng.standard_normal((B, 1, H, 512)).astype(np.float32))
    win = synth.bf16_round(rng.standard_normal((B, 128, 512)).astype(np.float32))
    ent = rng.standard_normal((B, N, 512)).astype(np.float32)
    if efmt == "bf16":
        ent = synth.bf16_round(ent)
    sink = rng.standard_normal(H).astype(np.float32)
    pos = np.array([[128 * N + 5000], [5000], [50]], np.int32)  # all / 39 entries / window only
    say(f"hca attn {efmt}")
    out = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = _lib.workspace(_lib.hca_attn_workspace_size(B, 1, H, N))
    _lib.hca_attn_decode(bf16(q), "bf16", bf16(win), "bf16", _lib.WIN_RING128, None, 128,
                         upload_rows(ent, efmt), efmt, N, 128, i32(pos), B, 1, H, f32(sink),
                         512 ** -0.5, cos, sin, out, "bf16", ws)
    got = to_np(out)
    entv = codec.store(ent, efmt)[1]
    for b in range(B):
        t = int(pos[b, 0])
        ref = A.hca_decode(q[b, 0].astype(np.float64), win[b].astype(np.float64), A.window_ids(t),
                           entv[b], sink, 512 ** -0.5, t, OM)
        close_bf16(got[b, 0], ref)


def test_hca_decode_many_units(tables):
    """Enough (chunk, unit) items that every work-group takes all 64 heads
    (the head tiles are split over two work-groups only for small grids):
    2 sequences x 32 causal queries over 4,096 entries, sampled queries
    checked."""
    cos, sin = tables
    B, Q, H, N = 2, 32, 64, 4096
    rng = np.random.default_rng(37)
    q = synth.bf16_round(rng.standard_normal((B, Q, H, 512)).astype(np.float32))
    win = synth.bf16_round(rng.standard_normal((B, 128, 512)).astype(np.float32))
    ent = synth.bf16_round(rng.standard_normal((B, N, 512)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    # every query sees a different prefix; the last ones see all entries
    pos = (128 * N - 1 - 4000 * np.arange(Q)[::-1]).astype(np.int32)
    pos = np.stack([pos, pos - 17]).astype(np.int32)
    say("hca attn many units")
    out = torch.empty((B, Q, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = _lib.workspace(_lib.hca_attn_workspace_size(B, Q, H, N))
    _lib.hca_attn_decode(bf16(q), "bf16", bf16(win), "bf16", _lib.WIN_RING128, None, 128,
                         upload_rows(ent, "bf16"), "bf16", N, 128, i32(pos), B, Q, H, f32(sink),
                         512 ** -0.5, cos, sin, out, "bf16", ws)
    got = to_np(out)
    for b, qq in [(0, 0), (0, Q - 1), (1, 5), (1, Q - 1)]:
        t = int(pos[b, qq])
        ref = A.hca_decode(q[b, qq].astype(np.float64), win[b].astype(np.float64),
                           A.window_ids(t), ent[b], sink, 512 ** -0.5, t, OM)
        close_bf16(got[b, qq], ref)


def test_f32_path_and_single_head_group(tables):
    cos, sin = tables
    B, H, N, k = 1, 16, 512, 64
    rng = np.random.default_rng(41)
    q = rng.standard_normal((B, 1, H, 512)).astype(np.float32)
    win = rng.standard_normal((B, 128, 512)).astype(np.float32)
    ent = rng.standard_normal((B, N, 512)).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    pos = np.array([[2047]], np.int32)
    ids = gen_ids(rng, N, k, N).reshape(1, 1, k)
    out = torch.empty((B, 1, H, 512), dtype=torch.float32, device="cuda")
    ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(B, 1, H, k))
    _lib.csa_sparse_attn_decode(f32(q), "f32", f32(win), "f32", _lib.WIN_RING128, None, 128,
                                f32(ent), "f32", N, i32(ids), k, i32(pos), B, 1, H, f32(sink),
                                512 ** -0.5, cos, sin, out, "f32", ws)
    ref = oracle_sparse(q[0, 0].astype(np.float64), win[0].astype(np.float64),
                        ent[0].astype(np.float64), ids[0, 0], sink, 2047)
    close_f32(to_np(out)[0, 0], ref)


def test_permutation_padding_and_determinism(tables):
    cos, sin = tables
    B, H, N, k = 2, 64, 2000, 512
    rng = np.random.default_rng(51)
    q = bf16(synth.bf16_round(rng.standard_normal((B, 1, H, 512)).astype(np.float32)))
    win = bf16(synth.bf16_round(rng.standard_normal((B, 128, 512)).astype(np.float32)))
    ent = upload_rows(rng.standard_normal((B, N, 512)).astype(np.float32), "fp8_mx32")
    sink = f32(rng.standard_normal(H).astype(np.float32))
    pos = i32(np.array([[8191], [8191]]))
    ids = np.stack([rng.choice(N, size=k, replace=False) for _ in range(B)]).astype(np.int32)

    def run(idx):
        kk = idx.shape[-1]
        out = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device="cuda")
        ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(B, 1, H, kk))
        _lib.csa_sparse_attn_decode(q, "bf16", win, "bf16", 0, None, 128, ent, "fp8_mx32", N,
                                    i32(idx.reshape(B, 1, kk)), kk, pos, B, 1, H, sink,
                                    512 ** -0.5, cos, sin, out, "bf16", ws)
        return to_np(out)

    a = run(ids)
    assert np.array_equal(a, run(ids))                     # bitwise run to run
    close_bf16(run(ids[:, ::-1].copy()), a)                # permutation
    padded = np.concatenate([ids, np.full((B, 100), -1, np.int32)], axis=1)
    close_bf16(run(padded), a)                             # -1 rows are absent


@pytest.mark.parametrize("Q,efmt", [(1, "fp4_e4m3_16"), (1, "fp8_mx32"), (20, "bf16")])
def test_shared_entries_layer_group(tables, Q, efmt):
    """csa_sparse_attn_decode_shared: L layers x B sequences in one launch,
    sharing B entry sets and top-k lists, each layer with its own q, window
    and sinks, equal bit for bit to one csa_sparse_attn_decode call per layer
    (20 queries per sequence take the 640-row chunks)."""
    cos, sin = tables
    B, L, H, N, k = 3, 4, 64, 2500, 512
    rng = np.random.default_rng(31 + Q)
    ent = rng.standard_normal((B, N, 512)).astype(np.float32)
    if efmt == "bf16":
        ent = synth.bf16_round(ent)
    ent_d = upload_rows(ent, efmt)
    q = synth.bf16_round(rng.standard_normal((L, B, Q, H, 512)).astype(np.float32))
    win = rng.standard_normal((L, B, 128, 512)).astype(np.float32)
    win_d = upload_rows(win.reshape(L * B, 128, 512), "fp8_mx32")
    sink = rng.standard_normal((L, H)).astype(np.float32)
    pos = (np.array([4 * N - 1, 300, 2000])[:, None] + np.arange(Q)[None, :] * 0).astype(np.int32)
    ids = np.stack([np.stack([gen_ids(rng, min((int(pos[b, i]) + 1) // 4, N), k, N)
                              for i in range(Q)]) for b in range(B)])        # [B, Q, k]
    ids_d = i32(ids)
    say(f"shared attn L={L} B={B} Q={Q} {efmt}")
    out = torch.empty((L * B, Q, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(L * B, Q, H, k))
    _lib.csa_sparse_attn_decode_shared(bf16(q.reshape(L * B, Q, H, 512)), "bf16", win_d, "fp8_mx32",
                                       ent_d, efmt, N, ids_d, k, i32(np.tile(pos, (L, 1))), L * B,
                                       Q, H, B, f32(sink), 512 ** -0.5, cos, sin, out, "bf16", ws)
    ws1 = _lib.workspace(_lib.csa_sparse_attn_workspace_size(B, Q, H, k))
    for lay in range(L):
        ref = torch.empty((B, Q, H, 512), dtype=torch.bfloat16, device="cuda")
        _lib.csa_sparse_attn_decode(bf16(q[lay]), "bf16", win_d[lay * B:(lay + 1) * B].contiguous(),
                                    "fp8_mx32", _lib.WIN_RING128, None, 128, ent_d, efmt, N, ids_d,
                                    k, i32(pos), B, Q, H, f32(sink[lay]), 512 ** -0.5, cos, sin,
                                    ref, "bf16", ws1)
        torch.cuda.synchronize()
        assert torch.equal(out[lay * B:(lay + 1) * B], ref), lay
    # ent_seqs must divide B
    with pytest.raises(_lib.CsaError):
        _lib.csa_sparse_attn_decode_shared(bf16(q.reshape(L * B, Q, H, 512)), "bf16", win_d,
                                           "fp8_mx32", ent_d, efmt, N, ids_d, k,
                                           i32(np.tile(pos, (L, 1))), L * B, Q, H, 5, f32(sink),
                                           512 ** -0.5, cos, sin, out, "bf16", ws)
