"""Indexer-score and fused top-k parity (GPU).

Scores: the library's float32 scores against the oracle's float64 scores on
the same bf16 / FP8 inputs, within an error bound derived from float32
accumulation (two dot-product levels: 128 dims, then the weighted head sum).
Indices: every returned list is checked for validity against the library's
own scores, and against the oracle's selection wherever the oracle's boundary
gap exceeds the score tolerance.
"""

import numpy as np
import pytest
import torch

from kv_cache_decode_csa_amd import _lib, synth
from oracle import codec, indexer
from oracle import topk as _TK

from gpu_util import bf16, check_selection, f32, i32, need_gpu, say, score_bound, upload_rows

pytestmark = pytest.mark.gpu

@pytest.mark.parametrize("kfmt,Hi,N", [("bf16", 32, 3000), ("bf16", 64, 3000),
                                        ("fp8_mx32", 32, 3000), ("fp8_mx32", 64, 3000),
                                        ("fp8_mx32", 64, 3001), ("bf16", 16, 1029),
                                        ("fp8_mx32", 16, 1029), ("fp8_mx32", 48, 2000)])
def test_scores_and_topk(kfmt, Hi, N):
    """Several work-groups per row, partial last steps, n_vis clamping; N = 3001
    puts the per-sequence key bases off 16-byte alignment (132-B rows)."""
    need_gpu()
    B, Q, k = 3, 2, 512
    w = synth.Workload(90, "t", B=B, ctx=4 * N, ratio=4, n_entries=N, Hi=Hi, key_fmt=kfmt)
    qi = synth.bf16_round(synth.normal_batched(w.seed, synth.T_QIDX, B, (Q, Hi, 128)))
    wi = synth.normal_batched(w.seed, synth.T_WIDX, B, (Q, Hi), (128 * Hi) ** -0.5)
    K = synth.index_keys(w)                                           # [B, N, 128] f32 values
    pos = np.array([[4 * N - 1, 2047], [5, 0], [601, 4 * N + 900]], np.int32)  # n_vis clamps
    say(f"index_topk {kfmt} Hi={Hi} N={N}")
    kdev = upload_rows(K, kfmt)
    out = torch.empty((B, Q, k), dtype=torch.int32, device="cuda")
    sc = torch.full((B, Q, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, Q, N, k))
    _lib.csa_index_topk(bf16(qi), "bf16", f32(wi), kdev, kfmt, i32(pos), 4, B, Q, Hi, N, k, out,
                        sc, ws)
    out = out.cpu().numpy()
    sc = sc.cpu().numpy()
    Kv = codec.store(K, kfmt)[1] if kfmt != "bf16" else K.astype(np.float64)
    for b in range(B):
        for qq in range(Q):
            nv = int(indexer.n_visible(pos[b, qq], 4, N))
            S_ref = indexer.scores(qi[b, qq].astype(np.float64), wi[b, qq], Kv[b], nv)
            tol = score_bound(qi[b, qq].astype(np.float64), wi[b, qq].astype(np.float64),
                              Kv[b][:nv])
            err = np.abs(sc[b, qq, :nv] - S_ref)
            assert np.all(err <= tol), (b, qq, err.max(), tol[err.argmax()])
            check_selection(out[b, qq], sc[b, qq], S_ref, tol, nv, k)


@pytest.mark.parametrize("Hi", [64, 32])
def test_many_queries_query_tiles(Hi):
    """12+ queries per sequence with bf16 keys (chunked prefill) take the
    query-tiled kernel: 21 queries (a ragged tile of 9), 70,000 keys (three key
    ranges, a partial last step), causal visibility per query including an
    empty one.  Scores match the oracle, are bit-identical to one-query calls
    (the per-query kernel), and nothing past a query's visible count is written."""
    need_gpu()
    B, Q, N, k = 2, 21, 70000, 512
    w = synth.Workload(91, "t", B=B, ctx=4 * N, ratio=4, n_entries=N, Hi=Hi, key_fmt="bf16")
    qi = synth.bf16_round(synth.normal_batched(w.seed, synth.T_QIDX, B, (Q, Hi, 128)))
    wi = synth.normal_batched(w.seed, synth.T_WIDX, B, (Q, Hi), (128 * Hi) ** -0.5)
    K = synth.index_keys(w)
    pos = np.stack([4 * N - Q - 40 + np.arange(Q), 1 + 37 * np.arange(Q)]).astype(np.int32)
    say(f"index_topk query tiles Hi={Hi}")
    kdev = upload_rows(K, "bf16")
    qd, wd = bf16(qi), f32(wi)
    out = torch.empty((B, Q, k), dtype=torch.int32, device="cuda")
    sc = torch.full((B, Q, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, Q, N, k))
    _lib.csa_index_topk(qd, "bf16", wd, kdev, "bf16", i32(pos), 4, B, Q, Hi, N, k, out, sc, ws)
    out = out.cpu().numpy()
    sc = sc.cpu().numpy()
    # one-query calls through the per-query kernel
    ws1 = _lib.workspace(_lib.csa_index_topk_workspace_size(1, 1, N, k))
    for b in range(B):
        for qq in range(Q):
            o1 = torch.empty((1, 1, k), dtype=torch.int32, device="cuda")
            s1 = torch.full((1, 1, N), float("nan"), dtype=torch.float32, device="cuda")
            _lib.csa_index_topk(qd[b, qq].contiguous(), "bf16", wd[b, qq].contiguous(),
                                kdev[b].contiguous(), "bf16", i32(pos[b, qq:qq + 1]), 4, 1, 1,
                                Hi, N, k, o1, s1, ws1)
            nv = int(indexer.n_visible(pos[b, qq], 4, N))
            s1 = s1.cpu().numpy()[0, 0]
            assert np.array_equal(s1[:nv].view(np.uint32), sc[b, qq, :nv].view(np.uint32)), (b, qq)
            assert np.all(np.isnan(sc[b, qq, nv:])), (b, qq)
            assert np.array_equal(o1.cpu().numpy()[0, 0], out[b, qq]), (b, qq)
            S_ref = indexer.scores(qi[b, qq].astype(np.float64), wi[b, qq], K[b], nv)
            tol = score_bound(qi[b, qq].astype(np.float64), wi[b, qq].astype(np.float64), K[b][:nv])
            err = np.abs(sc[b, qq, :nv] - S_ref)
            assert np.all(err <= tol), (b, qq, err.max())
            check_selection(out[b, qq], sc[b, qq], S_ref, tol, nv, k)


@pytest.mark.parametrize("Hi,N", [(64, 3000), (32, 5001)])
def test_fp4_keys_against_oracle(Hi, N):
    """FP4 indexer keys: MXFP4-MX32 rows (68 B), queries carrying MXFP4 values
    (exact in bf16); float32 scores against the oracle's scores of the decoded
    values, and the selection."""
    need_gpu()
    B, Q, k = 2, 2, 512
    w = synth.Workload(92, "t", B=B, ctx=4 * N, ratio=4, n_entries=N, Hi=Hi, key_fmt="fp4_mx32")
    K = synth.index_keys(w)
    qraw = synth.normal_batched(w.seed, synth.T_QIDX, B, (Q, Hi, 128))
    qi = codec.store(qraw, "fp4_mx32")[1].astype(np.float32)
    assert np.array_equal(synth.bf16_round(qi), qi)            # FP4 values are exact in bf16
    wi = synth.normal_batched(w.seed, synth.T_WIDX, B, (Q, Hi), (128 * Hi) ** -0.5)
    pos = np.array([[4 * N - 1, 2047], [5, 4 * N + 900]], np.int32)
    say(f"index_topk fp4_mx32 Hi={Hi} N={N}")
    kdev = upload_rows(K, "fp4_mx32")
    # the library's stored rows are the oracle codec's bytes
    assert np.array_equal(kdev.cpu().numpy(), codec.store(K, "fp4_mx32")[0])
    Kv = codec.store(K, "fp4_mx32")[1]
    out = torch.empty((B, Q, k), dtype=torch.int32, device="cuda")
    sc = torch.full((B, Q, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, Q, N, k))
    _lib.csa_index_topk(bf16(qi), "bf16", f32(wi), kdev, "fp4_mx32", i32(pos), 4, B, Q, Hi, N, k,
                        out, sc, ws)
    out = out.cpu().numpy()
    sc = sc.cpu().numpy()
    for b in range(B):
        for qq in range(Q):
            nv = int(indexer.n_visible(pos[b, qq], 4, N))
            S_ref = indexer.scores(qi[b, qq].astype(np.float64), wi[b, qq], Kv[b], nv)
            tol = score_bound(qi[b, qq].astype(np.float64), wi[b, qq].astype(np.float64),
                              Kv[b][:nv])
            err = np.abs(sc[b, qq, :nv] - S_ref)
            assert np.all(err <= tol), (b, qq, err.max())
            check_selection(out[b, qq], sc[b, qq], S_ref, tol, nv, k)


@pytest.mark.parametrize("Hi,N,bf16_scores", [(64, 3000, False), (32, 5001, False),
                                               (64, 4000, True), (16, 700, True)])
def test_fp4_queries_and_keys(Hi, N, bf16_scores):
    """FP4 queries and FP4 keys (MXFP4-MX32 rows of 68 B on both sides): the
    block-scaled FP4 MFMA path.  Scores against the oracle's scores of the
    decoded values within the float32 bound, the selection against the
    oracle's, and both against the call that takes the same queries as bf16
    values (the bf16 MFMA of the decoded values): E2M1 products are exact on
    both paths, so the scores agree within the float32 accumulation bound and
    the bf16-rounded scores' selections are checked as in the bf16 test."""
    need_gpu()
    B, Q, k = 2, 2, 512
    w = synth.Workload(94, "t", B=B, ctx=4 * N, ratio=4, n_entries=N, Hi=Hi, key_fmt="fp4_mx32")
    K = synth.index_keys(w)
    qraw = synth.normal_batched(w.seed, synth.T_QIDX, B, (Q, Hi, 128))
    qrows, qi = codec.store(qraw, "fp4_mx32")
    qi = qi.astype(np.float32)
    wi = synth.normal_batched(w.seed, synth.T_WIDX, B, (Q, Hi), (128 * Hi) ** -0.5)
    pos = np.array([[4 * N - 1, 2047], [5, 4 * N + 900]], np.int32)
    say(f"index_topk fp4 queries Hi={Hi} N={N} bf16_scores={bf16_scores}")
    kdev = upload_rows(K, "fp4_mx32")
    qdev = upload_rows(qraw, "fp4_mx32")
    assert np.array_equal(qdev.cpu().numpy(), qrows)            # the oracle codec's bytes
    Kv = codec.store(K, "fp4_mx32")[1]
    fn = _lib.csa_index_topk_bf16 if bf16_scores else _lib.csa_index_topk
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, Q, N, k))
    res = {}
    for qf, qa in (("fp4_mx32", qdev), ("bf16", bf16(qi))):
        out = torch.empty((B, Q, k), dtype=torch.int32, device="cuda")
        sc = torch.full((B, Q, N), float("nan"), dtype=torch.float32, device="cuda")
        fn(qa, qf, f32(wi), kdev, "fp4_mx32", i32(pos), 4, B, Q, Hi, N, k, out, sc, ws)
        res[qf] = (out.cpu().numpy(), sc.cpu().numpy())
    out, sc = res["fp4_mx32"]
    for b in range(B):
        for qq in range(Q):
            nv = int(indexer.n_visible(pos[b, qq], 4, N))
            S_ref = indexer.scores(qi[b, qq].astype(np.float64), wi[b, qq], Kv[b], nv)
            tol = score_bound(qi[b, qq].astype(np.float64), wi[b, qq].astype(np.float64),
                              Kv[b][:nv])
            if bf16_scores:
                # the bf16-rounded scores: one bf16 step beyond the float32 bound
                tol = tol + np.abs(S_ref) * 2.0 ** -8
                s32 = sc[b, qq, :nv]
                assert np.array_equal(codec.round_to_bf16(s32).astype(np.float32).view(np.uint32),
                                      s32.view(np.uint32))
                assert np.array_equal(out[b, qq], _TK.topk(s32, k, nv)), (b, qq)
            err = np.abs(sc[b, qq, :nv] - S_ref)
            assert np.all(err <= tol), (b, qq, err.max())
            check_selection(out[b, qq], sc[b, qq], S_ref, tol, nv, k)
            d = np.abs(sc[b, qq, :nv] - res["bf16"][1][b, qq, :nv])
            assert np.all(d <= 2 * tol), (b, qq, d.max())


@pytest.mark.parametrize("kfmt,Q", [("fp4_mx32", 2), ("fp8_mx32", 2), ("bf16", 13)])
def test_bf16_scores(kfmt, Q):
    """csa_index_topk_bf16 (every kernel: per-query FP4, split FP8, query-tiled
    bf16): its scores are the float32 call's scores rounded to bf16 (RNE), bit
    for bit, and its ids are exactly the oracle's top-k of those scores (ties,
    which the rounding makes common, go to the smaller index)."""
    need_gpu()
    B, N, Hi, k = 2, 4000, 64, 512
    w = synth.Workload(93, "t", B=B, ctx=4 * N, ratio=4, n_entries=N, Hi=Hi, key_fmt=kfmt)
    K = synth.index_keys(w)
    qi = synth.bf16_round(synth.normal_batched(w.seed, synth.T_QIDX, B, (Q, Hi, 128)))
    wi = synth.normal_batched(w.seed, synth.T_WIDX, B, (Q, Hi), (128 * Hi) ** -0.5)
    pos = (4 * N - 1 - 37 * np.arange(B * Q)).reshape(B, Q).astype(np.int32)
    say(f"index_topk_bf16 {kfmt} Q={Q}")
    kdev = upload_rows(K, kfmt)
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, Q, N, k))
    res = []
    for fn in (_lib.csa_index_topk, _lib.csa_index_topk_bf16):
        out = torch.empty((B, Q, k), dtype=torch.int32, device="cuda")
        sc = torch.full((B, Q, N), float("nan"), dtype=torch.float32, device="cuda")
        fn(bf16(qi), "bf16", f32(wi), kdev, kfmt, i32(pos), 4, B, Q, Hi, N, k, out, sc, ws)
        res.append((out.cpu().numpy(), sc.cpu().numpy()))
    (o32, s32), (o16, s16) = res
    for b in range(B):
        for qq in range(Q):
            nv = int(indexer.n_visible(pos[b, qq], 4, N))
            want = codec.round_to_bf16(s32[b, qq, :nv]).astype(np.float32)
            assert np.array_equal(s16[b, qq, :nv].view(np.uint32), want.view(np.uint32))
            assert np.array_equal(o16[b, qq], _TK.topk(s16[b, qq, :nv], k, nv)), (b, qq)


def test_without_score_output_matches():
    """out_scores is optional: the indices are the same either way."""
    need_gpu()
    B, N, Hi, k = 2, 5000, 64, 64
    rng = np.random.default_rng(4)
    qi = synth.bf16_round(rng.standard_normal((B, 1, Hi, 128)).astype(np.float32))
    wi = rng.standard_normal((B, 1, Hi)).astype(np.float32)
    K = rng.standard_normal((B, N, 128)).astype(np.float32)
    kd = upload_rows(K, "fp8_mx32")
    pos = i32(np.array([[4 * N - 1], [4 * N - 1]]))
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, 1, N, k))
    o1 = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    o2 = torch.empty_like(o1)
    sc = torch.empty((B, 1, N), dtype=torch.float32, device="cuda")
    _lib.csa_index_topk(bf16(qi), "bf16", f32(wi), kd, "fp8_mx32", pos, 4, B, 1, Hi, N, k, o1, sc,
                        ws)
    _lib.csa_index_topk(bf16(qi), "bf16", f32(wi), kd, "fp8_mx32", pos, 4, B, 1, Hi, N, k, o2,
                        None, ws)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("kfmt", ["bf16", "fp8_mx32"])
def test_batch_invariance(kfmt):
    """A sequence's selection and scores do not depend on its batch neighbours
    (the work-group split of a row depends on the batch)."""
    need_gpu()
    B, N, Hi, k = 5, 4000, 64, 512
    rng = np.random.default_rng(5)
    qi = synth.bf16_round(rng.standard_normal((B, 1, Hi, 128)).astype(np.float32))
    wi = rng.standard_normal((B, 1, Hi)).astype(np.float32)
    K = synth.bf16_round(rng.standard_normal((B, N, 128)).astype(np.float32))
    pos = np.full((B, 1), 4 * N - 1, np.int32)
    res = []
    for bs in (list(range(B)), [2]):
        ws = _lib.workspace(_lib.csa_index_topk_workspace_size(len(bs), 1, N, k))
        o = torch.empty((len(bs), 1, k), dtype=torch.int32, device="cuda")
        sc = torch.empty((len(bs), 1, N), dtype=torch.float32, device="cuda")
        _lib.csa_index_topk(bf16(qi[bs]), "bf16", f32(wi[bs]), upload_rows(K[bs], kfmt), kfmt,
                            i32(pos[bs]), 4, len(bs), 1, Hi, N, k, o, sc, ws)
        res.append((o.cpu().numpy(), sc.cpu().numpy()))
    assert np.array_equal(res[0][0][2], res[1][0][0])
    assert np.array_equal(res[0][1][2], res[1][1][0])


def test_f32_path():
    need_gpu()
    B, N, Hi, k = 1, 512, 4, 64
    rng = np.random.default_rng(6)
    qi = rng.standard_normal((B, 1, Hi, 128)).astype(np.float32)
    wi = (rng.standard_normal((B, 1, Hi)) * (128 * Hi) ** -0.5).astype(np.float32)
    K = rng.standard_normal((B, N, 128)).astype(np.float32)
    pos = np.array([[2047]], np.int32)
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, 1, N, k))
    o = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, 1, N), dtype=torch.float32, device="cuda")
    _lib.csa_index_topk(f32(qi), "f32", f32(wi), f32(K), "f32", i32(pos), 4, B, 1, Hi, N, k, o, sc,
                        ws)
    S_ref = indexer.scores(qi[0, 0].astype(np.float64), wi[0, 0], K[0].astype(np.float64), N)
    tol = score_bound(qi[0, 0].astype(np.float64), wi[0, 0].astype(np.float64),
                      K[0].astype(np.float64))
    assert np.all(np.abs(sc.cpu().numpy()[0, 0] - S_ref) <= tol)
    check_selection(o.cpu().numpy()[0, 0], sc.cpu().numpy()[0, 0], S_ref, tol, N, k)
