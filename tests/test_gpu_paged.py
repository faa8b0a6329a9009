"""The block cache (GPU): every paged call against its contiguous counterpart
on the same logical data, and against the oracle where a block is missing.

"DeepSeek-V4 deep dive" section 9.4: compressed entries and index keys live
in a pool of blocks found through per-sequence block tables, the window ring
and compressor slots in per-request state slots.  A paged call only changes
where rows are read or written, so its results must equal, bit for bit, the
contiguous call's on the rows gathered through the table (the oracle's
``paged.gather``).  Where the table leaves a visible block unallocated, the
paged index call scores its keys as zero keys and the attention calls drop its
rows; those cases are checked against the contiguous call on zeroed keys and
against the oracle's attention without those rows.
"""

import numpy as np
import pytest
import torch

from kv_cache_decode_csa_amd import _lib, synth
from oracle import attention as OA
from oracle import codec, indexer, rope
from oracle import paged as OP

from gpu_util import (bf16, check_selection, close_bf16, f32, i32, need_gpu, rope_tables, say,
                      score_bound, to_np, upload_rows)

pytestmark = pytest.mark.gpu

OM = rope.frequencies(160000.0)


def make_pool(logical, counts, bs, rng, spare=5, holes=()):
    """Scatter logical rows [B, Nmax, ...] (device) into a shuffled block pool.
    counts[b] entries of sequence b are placed; holes lists (b, j) blocks left
    unallocated (-1).  Returns (pool, table (device int32), table (host))."""
    B, Nmax = logical.shape[0], logical.shape[1]
    max_blocks = -(-Nmax // bs)
    n_blocks = sum(-(-int(c) // bs) for c in counts) + spare
    table = OP.allocate(counts, bs, n_blocks, rng, max_blocks=max_blocks)
    for b, j in holes:
        table[b, j] = -1
    pool = torch.zeros((n_blocks, bs) + tuple(logical.shape[2:]), dtype=logical.dtype,
                       device=logical.device)
    for b in range(B):
        for j in range(max_blocks):
            if table[b, j] >= 0:
                lo, hi = j * bs, min((j + 1) * bs, Nmax)
                pool[int(table[b, j]), :hi - lo] = logical[b, lo:hi]
    return pool, i32(table), table


# ------------------------------------------------------------------ index + top-k
@pytest.mark.parametrize("kfmt,bs,Hi,N", [("fp8_mx32", 32, 64, 3000), ("fp8_mx32", 64, 32, 2080),
                                          ("fp8_mx32", 128, 16, 1029), ("fp4_mx32", 32, 64, 3000),
                                          ("fp4q", 32, 64, 3000), ("fp4q", 64, 16, 1029),
                                          ("bf16", 32, 32, 2000), ("f32", 32, 8, 700)])
def test_index_topk_paged_equals_contiguous(kfmt, bs, Hi, N):
    """Several work-groups per row, ragged visible counts (n_vis not a multiple
    of 32 or of a step), bf16 and float32 scores; fp4q: FP4 keys with FP4
    queries (the block-scaled MFMA path)."""
    fp4q = kfmt == "fp4q"
    kfmt = "fp4_mx32" if fp4q else kfmt
    need_gpu()
    rng = np.random.default_rng(sum(map(ord, kfmt)) + bs)
    B, Q, k = 3, 2, 512
    Nmax = -(-N // bs) * bs
    w = synth.Workload(91, "t", B=B, ctx=4 * Nmax, ratio=4, n_entries=Nmax, Hi=Hi, key_fmt=kfmt)
    K = synth.index_keys(w)
    qf = "f32" if kfmt == "f32" else "bf16"
    qi = synth.bf16_round(synth.normal_batched(w.seed, synth.T_QIDX, B, (Q, Hi, 128)))
    wi = synth.normal_batched(w.seed, synth.T_WIDX, B, (Q, Hi), (128 * Hi) ** -0.5)
    pos = np.array([[4 * N - 1, 2047], [5, 4 * Nmax + 99], [4 * N - 1 - 4 * 37, 4 * 33 + 2]],
                   np.int32)
    kdev = upload_rows(K, kfmt)
    counts = [N, N, N]
    pool, tdev, _ = make_pool(kdev, counts, bs, rng)
    kt = _lib.make_block_table(tdev, bs, pool.shape[0])
    up = f32 if qf == "f32" else bf16
    qd, wd, pd = up(qi), f32(wi), i32(pos)
    if fp4q:
        qf, qd = "fp4_mx32", upload_rows(qi, "fp4_mx32")
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, Q, Nmax, k))
    for bf in (0, 1):
        say(f"index_topk_paged {kfmt} bs={bs} Hi={Hi} N={N} bf16_scores={bf}")
        o1 = torch.empty((B, Q, k), dtype=torch.int32, device="cuda")
        o2 = torch.empty_like(o1)
        s1 = torch.full((B, Q, Nmax), float("nan"), dtype=torch.float32, device="cuda")
        s2 = torch.full_like(s1, float("nan"))
        fn = _lib.csa_index_topk_bf16 if bf else _lib.csa_index_topk
        fn(qd, qf, wd, kdev, kfmt, pd, 4, B, Q, Hi, Nmax, k, o1, s1, ws)
        _lib.csa_index_topk_paged(qd, qf, wd, pool, kfmt, kt, pd, 4, B, Q, Hi, k, bf, o2, s2, ws)
        torch.cuda.synchronize()
        s1, s2 = s1.cpu().numpy(), s2.cpu().numpy()
        for b in range(B):
            for q in range(Q):
                nv = int(indexer.n_visible(pos[b, q], 4, Nmax))
                assert np.array_equal(s1[b, q, :nv].view(np.uint32), s2[b, q, :nv].view(np.uint32))
        assert torch.equal(o1, o2)


def test_index_topk_paged_oracle_and_holes():
    """FP8 keys, 32 per block: the paged scores against the oracle's scores of
    the keys gathered through the table; then two visible blocks of sequence
    1 left unallocated: their keys score exactly 0 and everything equals the
    contiguous call on keys zeroed there."""
    need_gpu()
    rng = np.random.default_rng(12)
    B, Q, Hi, k, bs = 2, 1, 64, 256, 32
    N = 4000
    Nmax = -(-N // bs) * bs
    w = synth.Workload(92, "t", B=B, ctx=4 * Nmax, ratio=4, n_entries=Nmax, Hi=Hi,
                       key_fmt="fp8_mx32")
    K = synth.index_keys(w)
    qi = synth.bf16_round(synth.normal_batched(w.seed, synth.T_QIDX, B, (Q, Hi, 128)))
    wi = synth.normal_batched(w.seed, synth.T_WIDX, B, (Q, Hi), (128 * Hi) ** -0.5)
    pos = np.array([[4 * N - 1], [4 * N - 3]], np.int32)
    kdev = upload_rows(K, "fp8_mx32")
    holes = [(1, 3), (1, 70)]
    pool, tdev, table = make_pool(kdev, [N, N], bs, rng, holes=holes)
    kt = _lib.make_block_table(tdev, bs, pool.shape[0])
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, Q, Nmax, k))
    out = torch.empty((B, Q, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Q, Nmax), dtype=torch.float32, device="cuda")
    say("index_topk_paged holes")
    _lib.csa_index_topk_paged(bf16(qi), "bf16", f32(wi), pool, "fp8_mx32", kt, i32(pos), 4, B, Q,
                              Hi, k, 0, out, sc, ws)
    torch.cuda.synchronize()
    out_h, sc_h = out.cpu().numpy(), sc.cpu().numpy()
    pool_h = pool.cpu().numpy()
    for b in range(B):
        nv = int(indexer.n_visible(pos[b, 0], 4, Nmax))
        rows, valid = OP.gather(pool_h, table[b], bs, np.arange(nv))
        Kv = codec.load(rows, "fp8_mx32", 128)
        Kv[~valid] = 0.0
        q64, w64 = qi[b, 0].astype(np.float64), wi[b, 0].astype(np.float64)
        S_ref = indexer.scores(q64, w64, Kv, nv)
        tol = score_bound(q64, w64, Kv)
        err = np.abs(sc_h[b, 0, :nv] - S_ref)
        assert np.all(err <= tol), (b, err.max())
        check_selection(out_h[b, 0], sc_h[b, 0], S_ref, tol, nv, k)
        if b == 1:
            for _, j in holes:
                assert np.all(sc_h[b, 0, j * bs:(j + 1) * bs] == 0.0)
    kz = kdev.clone()
    for b, j in holes:
        kz[b, j * bs:(j + 1) * bs] = 0
    o2 = torch.empty_like(out)
    s2 = torch.empty_like(sc)
    _lib.csa_index_topk(bf16(qi), "bf16", f32(wi), kz, "fp8_mx32", i32(pos), 4, B, Q, Hi, Nmax, k,
                        o2, s2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, o2)
    for b in range(B):
        nv = int(indexer.n_visible(pos[b, 0], 4, Nmax))
        assert np.array_equal(sc_h[b, 0, :nv].view(np.uint32),
                              s2.cpu().numpy()[b, 0, :nv].view(np.uint32))


# ------------------------------------------------------------------ attention
def _slots(B, n_slots, rng):
    return rng.permutation(n_slots)[:B].astype(np.int32)


@pytest.mark.parametrize("Q,H,qf,ef,bs,B,N", [(1, 64, "bf16", "fp8_mx32", 32, 3, 1500),
                                              (1, 32, "bf16", "fp4_e4m3_16", 64, 3, 1500),
                                              (16, 64, "bf16", "fp8_mx32", 32, 3, 1500),
                                              (16, 32, "bf16", "bf16", 32, 3, 1500),
                                              (1, 16, "f32", "f32", 32, 3, 1500),
                                              (1, 64, "bf16", "fp8_mx32", 32, 70, 600)])
def test_sparse_attn_paged_equals_contiguous(Q, H, qf, ef, bs, B, N):
    """64-row chunks (one query), 640-row chunks (16 queries; 64 heads take the
    all-heads kernel), the float32 kernel, and one work-group per whole list
    (70 sequences of 64 heads).  Ids include -1, ids past Nmax and ids in an
    unallocated block; those are absent, as -1 is in the contiguous call."""
    need_gpu()
    rng = np.random.default_rng(Q * 100 + H)
    k = 512
    Nmax = -(-N // bs) * bs
    E = rng.standard_normal((B, Nmax, 512)).astype(np.float32)
    win = rng.standard_normal((B, 128, 512)).astype(np.float32)
    q = rng.standard_normal((B, Q, H, 512)).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    pos = (4 * N - 1 - rng.integers(0, 400, size=(B, Q))).astype(np.int32)
    ids = rng.integers(0, N, size=(B, Q, k)).astype(np.int32)
    ids[:, :, 5] = -1
    ids[:, :, 7] = Nmax + 3
    hole = (1, 2)                                  # sequence 1, block 2
    ids[1, :, 9] = hole[1] * bs + 1
    wf = ef if ef != "f32" else "f32"
    edev, wdev = upload_rows(E, ef), upload_rows(win, wf)
    pool, tdev, _ = make_pool(edev, [N] * B, bs, rng, holes=[hole])
    et = _lib.make_block_table(tdev, bs, pool.shape[0])
    n_slots = B + 4
    slot = _slots(B, n_slots, rng)
    wpool = torch.zeros((n_slots,) + tuple(wdev.shape[1:]), dtype=wdev.dtype, device="cuda")
    for b in range(B):
        wpool[int(slot[b])] = wdev[b]
    cos, sin = rope_tables(1 << 16, yarn=False)
    qd = (f32 if qf == "f32" else bf16)(q if qf == "f32" else synth.bf16_round(q))
    of = "f32" if qf == "f32" else "bf16"
    ids_ref = ids.copy()
    in_hole = (ids_ref[1] >= 0) & (ids_ref[1] < Nmax) & (ids_ref[1] // bs == hole[1])
    ids_ref[1][in_hole] = -1                       # rows of the unallocated block are absent
    assert in_hole.any()
    ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(B, Q, H, k))
    o1 = torch.empty((B, Q, H, 512), dtype=torch.float32 if of == "f32" else torch.bfloat16,
                     device="cuda")
    o2 = torch.empty_like(o1)
    say(f"sparse_attn_paged Q={Q} H={H} {qf}/{ef} bs={bs}")
    _lib.csa_sparse_attn_decode(qd, qf, wdev, wf, _lib.WIN_RING128, None, 128, edev, ef, Nmax,
                                i32(ids_ref), k, i32(pos), B, Q, H, f32(sink), 512 ** -0.5, cos,
                                sin, o1, of, ws)
    _lib.csa_sparse_attn_decode_paged(qd, qf, wpool, wf, i32(slot), n_slots, pool, ef, et,
                                      i32(ids), k, i32(pos), B, Q, H, f32(sink), 512 ** -0.5, cos,
                                      sin, o2, of, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16) if of == "bf16" else o1.view(torch.int32),
                       o2.view(torch.int16) if of == "bf16" else o2.view(torch.int32))


def test_sparse_attn_paged_slot_outside_pool():
    """A sequence whose window slot lies outside the pool attends over its
    entries alone (oracle: every window id absent)."""
    need_gpu()
    rng = np.random.default_rng(5)
    B, Q, H, k, N, bs = 2, 1, 64, 64, 300, 32
    Nmax = -(-N // bs) * bs
    E = synth.bf16_round(rng.standard_normal((B, Nmax, 512)).astype(np.float32))
    win = synth.bf16_round(rng.standard_normal((B, 128, 512)).astype(np.float32))
    q = synth.bf16_round(rng.standard_normal((B, Q, H, 512)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    pos = np.array([[4 * N - 1], [4 * N - 2]], np.int32)
    ids = np.stack([rng.permutation(N)[:k] for _ in range(B)]).astype(np.int32)[:, None]
    edev, wdev = upload_rows(E, "bf16"), upload_rows(win, "bf16")
    pool, tdev, table = make_pool(edev, [N] * B, bs, rng)
    et = _lib.make_block_table(tdev, bs, pool.shape[0])
    slot = np.array([1, 7], np.int32)             # 7 is outside a pool of 2 slots
    wpool = torch.zeros((2, 128, 512), dtype=torch.bfloat16, device="cuda")
    wpool[1] = wdev[0]
    cos, sin = rope_tables(1 << 14, yarn=False)
    ws = _lib.workspace(_lib.csa_sparse_attn_workspace_size(B, Q, H, k))
    out = torch.empty((B, Q, H, 512), dtype=torch.float32, device="cuda")
    say("sparse_attn_paged slot outside the pool")
    _lib.csa_sparse_attn_decode_paged(bf16(q), "bf16", wpool, "bf16", i32(slot), 2, pool, "bf16",
                                      et, i32(ids), k, i32(pos), B, Q, H, f32(sink), 512 ** -0.5,
                                      cos, sin, out, "f32", ws)
    torch.cuda.synchronize()
    out = to_np(out)
    pool_h = codec.bf16_bits_to_f64(pool.view(torch.int16).cpu().numpy().view(np.uint16))
    for b in range(B):
        t = int(pos[b, 0])
        rows, _ = OP.gather(pool_h, table[b], bs, np.arange(N))
        wids = OA.window_ids(t) if b == 0 else -np.ones(128, np.int64)
        ref = OA.sparse_decode(q[b, 0].astype(np.float64), win[b].astype(np.float64), wids, rows,
                               ids[b, 0], sink.astype(np.float64), 512 ** -0.5, t, OM)
        close_bf16(out[b, 0], ref)


@pytest.mark.parametrize("H,qf", [(64, "bf16"), (128, "bf16"), (16, "f32")])
def test_hca_attn_paged(H, qf):
    """HCA: one entry per 128-token block (block_entries 1), every visible
    entry through the table: 64 heads take the all-heads kernel, 128 heads the
    head-group kernel, float32 queries the float32 kernel.  Equal to the
    contiguous call bit for bit; with one entry unallocated, equal to the
    oracle without that row."""
    need_gpu()
    rng = np.random.default_rng(H)
    B, Q, N, bs = 3, 1, 1500, 1
    ef = "f32" if qf == "f32" else "fp8_mx32"
    E = rng.standard_normal((B, N, 512)).astype(np.float32)
    win = rng.standard_normal((B, 128, 512)).astype(np.float32)
    q = rng.standard_normal((B, Q, H, 512)).astype(np.float32)
    if qf == "bf16":
        q = synth.bf16_round(q)
    sink = rng.standard_normal(H).astype(np.float32)
    pos = np.array([[128 * N - 1], [128 * 1000 + 77], [128 * 700 - 1]], np.int32)
    edev, wdev = upload_rows(E, ef), upload_rows(win, ef)
    cos, sin = rope_tables(1 << 18, yarn=False)
    up = f32 if qf == "f32" else bf16
    of = "f32"
    ws = _lib.workspace(_lib.hca_attn_workspace_size(B, Q, H, N))
    slot = np.array([2, 0, 3], np.int32)
    wpool = torch.zeros((4,) + tuple(wdev.shape[1:]), dtype=wdev.dtype, device="cuda")
    for b in range(B):
        wpool[int(slot[b])] = wdev[b]
    for holes in ([], [(0, 345)]):
        pool, tdev, table = make_pool(edev, [N] * B, bs, rng, holes=holes)
        et = _lib.make_block_table(tdev, bs, pool.shape[0])
        o1 = torch.empty((B, Q, H, 512), dtype=torch.float32, device="cuda")
        o2 = torch.empty_like(o1)
        say(f"hca_attn_paged H={H} {qf} holes={holes}")
        _lib.hca_attn_decode_paged(up(q), qf, wpool, ef, i32(slot), 4, pool, ef, et, 128, i32(pos),
                                   B, Q, H, f32(sink), 512 ** -0.5, cos, sin, o2, of, ws)
        torch.cuda.synchronize()
        if not holes:
            _lib.hca_attn_decode(up(q), qf, wdev, ef, _lib.WIN_RING128, None, 128, edev, ef, N, 128,
                                 i32(pos), B, Q, H, f32(sink), 512 ** -0.5, cos, sin, o1, of, ws)
            torch.cuda.synchronize()
            assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
            continue
        got = to_np(o2)
        Ev = codec.load(edev.cpu().numpy(), ef, 512) if ef != "f32" else E.astype(np.float64)
        Wv = codec.load(wdev.cpu().numpy(), ef, 512) if ef != "f32" else win.astype(np.float64)
        b, e = holes[0]
        t = int(pos[b, 0])
        ids = OA.hca_ids(t, 128, n_max=N).copy()
        ids[ids == e] = -1
        ref = OA.sparse_decode(q[b, 0].astype(np.float64), Wv[b], OA.window_ids(t), Ev[b], ids,
                               sink.astype(np.float64), 512 ** -0.5, t, OM)
        if qf == "f32":
            err = np.abs(got[b, 0] - ref)
            assert np.all(err <= 1e-5 + 1e-5 * np.abs(ref)), err.max()
        else:
            close_bf16(got[b, 0], ref)


# ------------------------------------------------------------------ compressor
def _comp_setup(rng, B, dim, ratio, d, fmt):
    co = 2 if ratio == 4 else 1
    wkv = synth.bf16_round((rng.standard_normal((co * d, dim)) * 0.02).astype(np.float32))
    wg = synth.bf16_round((rng.standard_normal((co * d, dim)) * 0.02).astype(np.float32))
    ape = (rng.standard_normal((ratio, co * d)) * 0.02).astype(np.float32)
    up = bf16 if fmt == "bf16" else f32
    return up(wkv), up(wg), f32(ape), f32(np.ones(d, np.float32)), co


@pytest.mark.parametrize("ratio,d,rotate,efmt,fmt,bs", [(4, 512, 0, "fp8_mx32", "bf16", 32),
                                                        (4, 128, 1, "fp8_mx32", "bf16", 32),
                                                        (128, 512, 0, "fp8_mx32", "bf16", 1),
                                                        (4, 512, 0, "f32", "f32", 64)])
def test_compress_paged_equals_contiguous(ratio, d, rotate, efmt, fmt, bs):
    """A 600-token prompt in one call, then single-token calls across block
    boundaries (bf16: the fused decode kernels), with entries through a block
    table and the slot state in a pool of slots: the gathered entries and the
    slot states equal the contiguous calls' bit for bit.  One sequence's slot
    lies outside the pool: nothing of it is read or written."""
    need_gpu()
    rng = np.random.default_rng(ratio + d)
    B, dim, T0, steps = 3, 512, 600, 9
    wkv, wg, ape, nw, co = _comp_setup(rng, B, dim, ratio, d, fmt)
    cos, sin = rope_tables(1 << 12, yarn=False)
    n_cap = (T0 + steps) // ratio + 1
    Nmax = -(-n_cap // bs) * bs
    rb = _lib.kv_row_bytes(efmt, d)
    shape = (co * ratio, co * d)
    # contiguous
    ent1 = torch.zeros((B, Nmax, rb), dtype=torch.uint8, device="cuda")
    kv1 = torch.zeros((B,) + shape, dtype=torch.float32, device="cuda")
    sc1 = torch.full_like(kv1, float("-inf"))
    # paged: entries in a shuffled pool, state in slots (sequence 2 outside the pool)
    table = OP.allocate([Nmax] * B, bs, B * (Nmax // bs) + 3, rng)
    tdev = i32(table)
    pool = torch.zeros((table.max() + 4, bs, rb), dtype=torch.uint8, device="cuda")
    n_slots = 4
    slot = np.array([3, 1, 9], np.int32)
    kv2 = torch.zeros((n_slots,) + shape, dtype=torch.float32, device="cuda")
    sc2 = torch.full_like(kv2, float("-inf"))
    up = bf16 if fmt == "bf16" else f32
    x_all = rng.standard_normal((B, T0 + steps, dim)).astype(np.float32)
    if fmt == "bf16":
        x_all = synth.bf16_round(x_all)

    slot_dev = i32(slot)

    def call(x, start, paged):
        # the args hold raw pointers: every tensor they name stays referenced
        # until the call has been enqueued
        sp = i32(np.asarray(start, np.int32))
        xd = up(x)
        kw = dict(B=B, T=x.shape[1], dim=dim, ratio=ratio, head_dim=d, rotate=rotate, x=xd,
                  x_fmt=fmt, w_kv=wkv, w_gate=wg, w_fmt=fmt, ape=ape, norm_w=nw, eps=1e-6,
                  rope_cos=cos, rope_sin=sin, start_pos=sp, entry_fmt=efmt)
        if paged:
            a = _lib.make_compress_args(**kw, kv_state=kv2, score_state=sc2, entries=pool,
                                        block_table=tdev, block_entries=bs,
                                        pool_blocks=pool.shape[0], state_slot=slot_dev)
        else:
            a = _lib.make_compress_args(**kw, kv_state=kv1, score_state=sc1, entries=ent1,
                                        entries_cap=Nmax)
        _lib.csa_compress(a, _lib.workspace(_lib.csa_compress_workspace_size(a)))

    say(f"compress paged r={ratio} d={d} {efmt} {fmt} bs={bs}")
    for paged in (False, True):
        call(x_all[:, :T0], [0] * B, paged)
        for s in range(steps):
            call(x_all[:, T0 + s:T0 + s + 1], [T0 + s] * B, paged)
    torch.cuda.synchronize()
    e1 = ent1.cpu().numpy()
    pool_h = pool.cpu().numpy()
    n_done = (T0 + steps) // ratio
    for b in range(B):
        rows, valid = OP.gather(pool_h, table[b], bs, np.arange(n_done))
        if b == 2:                                 # skipped: its blocks hold zeros
            assert not rows.any()
            continue
        assert valid.all() and np.array_equal(rows, e1[b, :n_done])
        assert torch.equal(kv2[int(slot[b])], kv1[b]) and torch.equal(sc2[int(slot[b])], sc1[b])
    assert not (kv2[0] != 0).any() and torch.isinf(sc2[0]).all()   # the unused slot


def test_compress_many_paged_decode():
    """The fused single-token path of a CSA layer (main 512-d FP8 entries and
    128-d rotated FP8 index keys in one call), paged, over 40 steps from
    position 1000 with state continued from a contiguous prompt."""
    need_gpu()
    rng = np.random.default_rng(77)
    B, dim, T0, steps = 4, 1024, 1000, 40
    cos, sin = rope_tables(1 << 12, yarn=False)
    specs = [(512, 0), (128, 1)]
    mods = [_comp_setup(rng, B, dim, 4, d, "bf16") for d, _ in specs]
    x_all = synth.bf16_round(rng.standard_normal((B, T0 + steps, dim)).astype(np.float32))
    Nmax = 32 * ((T0 + steps) // 4 // 32 + 1)
    slot = np.array([5, 2, 0, 3], np.int32)
    bufs = []
    for (d, rot), (wkv, wg, ape, nw, co) in zip(specs, mods):
        rb = _lib.kv_row_bytes("fp8_mx32", d)
        shape = (8, 2 * d)
        ent1 = torch.zeros((B, Nmax, rb), dtype=torch.uint8, device="cuda")
        kv1 = torch.zeros((B,) + shape, dtype=torch.float32, device="cuda")
        sc1 = torch.full_like(kv1, float("-inf"))
        table = OP.allocate([Nmax] * B, 32, B * Nmax // 32 + 2, rng)
        pool = torch.zeros((B * Nmax // 32 + 2, 32, rb), dtype=torch.uint8, device="cuda")
        kv2 = torch.zeros((6,) + shape, dtype=torch.float32, device="cuda")
        sc2 = torch.full_like(kv2, float("-inf"))
        bufs.append(dict(ent1=ent1, kv1=kv1, sc1=sc1, table=table, tdev=i32(table), pool=pool,
                         kv2=kv2, sc2=sc2, d=d, rot=rot, w=(wkv, wg, ape, nw)))

    slot_dev = i32(slot)

    def args(x, start, paged):
        """The calls' args and the device tensors they point to (kept
        referenced by the caller until the calls are enqueued)."""
        xd = bf16(x)
        sp = i32(np.asarray(start, np.int32))
        out = []
        for bu in bufs:
            wkv, wg, ape, nw = bu["w"]
            kw = dict(B=B, T=x.shape[1], dim=dim, ratio=4, head_dim=bu["d"], rotate=bu["rot"],
                      x=xd, x_fmt="bf16", w_kv=wkv, w_gate=wg, w_fmt="bf16", ape=ape,
                      norm_w=nw, eps=1e-6, rope_cos=cos, rope_sin=sin, start_pos=sp,
                      entry_fmt="fp8_mx32")
            if paged:
                out.append(_lib.make_compress_args(**kw, kv_state=bu["kv2"], score_state=bu["sc2"],
                                                   entries=bu["pool"], block_table=bu["tdev"],
                                                   block_entries=32,
                                                   pool_blocks=bu["pool"].shape[0],
                                                   state_slot=slot_dev))
            else:
                out.append(_lib.make_compress_args(**kw, kv_state=bu["kv1"], score_state=bu["sc1"],
                                                   entries=bu["ent1"], entries_cap=Nmax))
        return out, (xd, sp)

    say("compress_many paged decode")
    for paged in (False, True):
        a, keep = args(x_all[:, :T0], [0] * B, paged)
        for ai in a:
            _lib.csa_compress(ai, _lib.workspace(_lib.csa_compress_workspace_size(ai)))
        for s in range(steps):
            a, keep = args(x_all[:, T0 + s:T0 + s + 1], [T0 + s] * B, paged)
            _lib.csa_compress_many(a, _lib.workspace(_lib.csa_compress_many_workspace_size(a)))
        del keep
    torch.cuda.synchronize()
    n_done = (T0 + steps) // 4
    for bu in bufs:
        e1 = bu["ent1"].cpu().numpy()
        ph = bu["pool"].cpu().numpy()
        for b in range(B):
            rows, valid = OP.gather(ph, bu["table"][b], 32, np.arange(n_done))
            assert valid.all() and np.array_equal(rows, e1[b, :n_done])
            assert torch.equal(bu["kv2"][int(slot[b])], bu["kv1"][b])
            assert torch.equal(bu["sc2"][int(slot[b])], bu["sc1"][b])
