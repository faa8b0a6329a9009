"""Pins for the oracle's indexer, top-k, attention and cache arithmetic (CPU only)."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import cache_bytes as CB
from oracle import compressor, indexer, rope
from oracle import topk as TK

OM = rope.frequencies(160000.0, rope.V4_YARN)
SCALE = 512 ** -0.5


# ----------------------------------------------------------------------------- selection

def test_index_selection_example(golden):
    g = golden["index_selection"]
    n = indexer.n_visible(g["t"], g["ratio"])
    assert n == g["visible"]
    sel = TK.topk(np.array(g["scores"], np.float32), g["k"], n)
    assert list(sel) == g["topk"]
    w = A.window_ids(g["t"], "linear", 0, window=g["window"])
    assert (w[0], w[-1]) == (g["window_first"], g["window_last"])
    assert len(w) + len(sel) == g["keys_total"]


def test_visibility_counts(golden):
    g = golden["visibility"]
    assert indexer.n_visible(10000, 4) == g["t_10000_blocks"]
    assert indexer.n_visible(9999, 4) == g["t_9999_blocks"]
    assert CB.sparsity_start(1024) == g["sparsity_start_pro"]
    assert indexer.n_visible(g["sparsity_start_pro"], 4) == g["visible_at_start_pro"]
    assert indexer.n_visible(g["sparsity_start_pro"] - 1, 4) == 1024
    assert CB.sparsity_start(512) == g["sparsity_start_flash"]
    assert indexer.n_visible(g["sparsity_start_flash"], 4) == g["visible_at_start_flash"]
    assert 128 + min(1024, indexer.n_visible(10000, 4)) == g["pro_keys_t10000"]
    assert len(A.hca_ids(10000)) == g["hca_entries_t10000"]
    assert len(A.hca_ids(10000)) + 128 == g["hca_keys_t10000"]


def test_topk_matches_bruteforce():
    rng = np.random.default_rng(0)
    for trial in range(60):
        n = int(rng.integers(1, 40))
        s = rng.choice(np.array([-1.5, -0.0, 0.0, 0.5, 0.5, 2.0, np.nan], np.float32), size=n)
        s = np.where(rng.random(n) < 0.5, s, rng.standard_normal(n).astype(np.float32))
        k = int(rng.integers(1, 50))
        nv = int(rng.integers(0, n + 1))
        np.testing.assert_array_equal(TK.topk(s, k, nv), TK.topk_bruteforce(s, k, nv))


def test_topk_padding_and_signed_zero():
    s = np.array([0.0, -0.0, 1.0, -0.0], np.float32)
    np.testing.assert_array_equal(TK.topk(s, 6), [2, 0, 1, 3, -1, -1])
    np.testing.assert_array_equal(TK.topk(s, 3, n_vis=0), [-1, -1, -1])


def test_scores_match_loops_and_hadamard_invariance():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((4, 128))
    w = rng.standard_normal(4)
    K = rng.standard_normal((9, 128))
    s = indexer.scores(q, w, K, 7)
    np.testing.assert_allclose(s, indexer.scores_loop(q, w, K, 7), rtol=1e-12, atol=1e-12)
    H = compressor.hadamard(128) / math.sqrt(128)
    s2 = indexer.scores(q @ H.T, w, K @ H.T, 7)
    np.testing.assert_allclose(s2, s, rtol=1e-12, atol=1e-12)
    assert len(s) == 7


# ----------------------------------------------------------------------------- attention

def test_sink_worked_example(golden):
    g = golden["sink"]
    H, D = 1, 512
    rows = np.zeros((3, D))
    rows[0, 0] = rows[1, 1] = rows[2, 2] = 1.0
    q = np.zeros((H, D))
    q[0, :3] = np.array(g["logits"]) / SCALE
    o = A.attend(q, rows, np.ones(3, bool), np.array([g["sink"]], float), SCALE, 0, OM)
    np.testing.assert_allclose(o[0, :3], g["weights_with_sink"], atol=0.5e-3)
    assert abs(o[0, :3].sum() - g["sum_with_sink"]) < 0.5e-3
    o = A.attend(q, rows, np.ones(3, bool), np.array([-np.inf]), SCALE, 0, OM)
    np.testing.assert_allclose(o[0, :3], g["weights_no_sink"], atol=0.5e-3)


def test_attention_equals_library_sdpa():
    rng = np.random.default_rng(2)
    H, n = 8, 37
    q = rng.standard_normal((H, 512))
    C = rng.standard_normal((n, 512))
    o = A.attend(q, C, np.ones(n, bool), np.full(H, -np.inf), SCALE, 0, OM)
    tq = torch.from_numpy(q)[None, :, None, :]
    tk = torch.from_numpy(C)[None, None].expand(1, H, n, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tk, scale=SCALE)
    np.testing.assert_allclose(o, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_ratio1_topk_all_equals_dense_attention():
    """m = 1 compression with top-k = all visible entries equals dense attention."""
    rng = np.random.default_rng(3)
    dim, T, H = 8, 40, 4
    wkv = rng.standard_normal((512, dim))
    x = rng.standard_normal((T, dim))
    out, _ = compressor.compress_bulk(x, 0, wkv, np.zeros((512, dim)), np.zeros((1, 512)),
                                      np.ones(512), OM, 1, 512)
    E = np.stack([out[i] for i in range(T)])
    t = T - 1
    n = indexer.n_visible(t, 1)
    sel = TK.topk(rng.standard_normal(n).astype(np.float32), n + 5, n)
    assert sorted(sel[:n]) == list(range(n)) and np.all(sel[n:] == -1)
    q = rng.standard_normal((H, 512))
    no_win = -np.ones(128, np.int64)
    o = A.sparse_decode(q, np.zeros((128, 512)), no_win, E, sel, np.full(H, -np.inf), SCALE,
                        t, OM)
    # dense reference through the library routine on the rotated query
    qr = rope.rotate(q, t, OM)
    tk = torch.from_numpy(E)[None, None].expand(1, H, n, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qr)[None, :, None, :], tk, tk, scale=SCALE)[0, :, 0].numpy()
    np.testing.assert_allclose(o, rope.rotate(ref, t, OM, inverse=True), rtol=1e-11, atol=1e-12)


def test_window_plus_entries_is_dense_over_concatenation_with_duplicates():
    rng = np.random.default_rng(4)
    H = 4
    win = rng.standard_normal((128, 512))
    E = rng.standard_normal((20, 512))
    E[3] = win[7]  # a duplicate row (raw and pooled copies of the same content)
    t = 300
    wid = A.window_ids(t)
    sel = np.array([3, 11, 3, -1, 0], np.int32)
    q = rng.standard_normal((H, 512))
    sink = rng.standard_normal(H)
    o = A.sparse_decode(q, win, wid, E, sel, sink, SCALE, t, OM)
    rows = np.concatenate([win[wid], E[[3, 11, 3, 0]]])
    o2 = A.attend(q, rows, np.ones(len(rows), bool), sink, SCALE, t, OM)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)


def test_shift_invariance():
    rng = np.random.default_rng(5)
    H, n = 4, 9
    u = rng.standard_normal((n, 512))
    ppos = rng.integers(0, 500, size=n)
    q = rng.standard_normal((H, 512))
    sink = rng.standard_normal(H)
    outs = []
    for delta in (0, 12345, 700000):
        rows = np.stack([rope.rotate(u[j], ppos[j] + delta, OM) for j in range(n)])
        outs.append(A.attend(q, rows, np.ones(n, bool), sink, SCALE, 600 + delta, OM))
    np.testing.assert_allclose(outs[1], outs[0], atol=1e-9)
    np.testing.assert_allclose(outs[2], outs[0], atol=1e-9)


def test_permutation_and_padding_invariance():
    rng = np.random.default_rng(6)
    H = 4
    win = rng.standard_normal((128, 512))
    E = rng.standard_normal((50, 512))
    q = rng.standard_normal((H, 512))
    sink = rng.standard_normal(H)
    t = 50
    wid = A.window_ids(t)
    assert np.sum(wid == -1) == 128 - 51
    sel = np.array([5, 17, 2, 44, 30], np.int32)
    base = A.sparse_decode(q, win, wid, E, sel, sink, SCALE, t, OM)
    perm = A.sparse_decode(q, win, wid, E, sel[::-1], sink, SCALE, t, OM)
    pad = A.sparse_decode(q, win, wid, E, np.array([5, -1, 17, 2, -1, 44, 30], np.int32), sink,
                          SCALE, t, OM)
    np.testing.assert_allclose(perm, base, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(pad, base, rtol=1e-12, atol=1e-13)
    empty = A.sparse_decode(q, win, -np.ones(128, np.int64), E, -np.ones(4, np.int32), sink,
                            SCALE, t, OM)
    np.testing.assert_array_equal(empty, 0.0)


def test_hca_key_counts(golden):
    g = golden["hca_t1000"]
    ids = A.hca_ids(1000)
    assert len(ids) == g["entries"] and ids[-1] * 128 == g["last_entry_rope_pos"]
    w = A.window_ids(1000, "linear")
    assert w[0] == g["window_first"] and len(ids) + len(w) == g["keys"]
    assert 1000 - (len(ids) * 128) + 1 == g["unfinished"]
    k = golden["keys_per_query"]
    for ctx, want in k["hca"].items():
        assert CB.keys_per_query("hca", int(ctx)) == want
    assert CB.keys_per_query("csa", 1 << 20, 1024) == k["csa_pro_1m"]
    assert CB.keys_per_query("csa", 1 << 20, 512) == k["csa_flash_1m"]


# ----------------------------------------------------------------------------- cache bytes

def test_cache_arithmetic(golden):
    g = golden["cache_bytes"]
    assert CB.naive_gqa_bytes_per_token(43) == g["naive_flash_per_token"]
    assert CB.hca_naive_bytes_per_token_layer() == g["hca_naive_per_token_layer"]
    assert CB.fp8_mx32_row_bytes() == g["fp8_row"] and CB.fp4_e4m3_16_row_bytes() == g["fp4_row"]
    assert CB.mla_bytes_per_token() == g["v2_mla_per_token"]
    assert CB.naive_mha_bytes_per_token() == g["v2_naive_per_token"]
    assert CB.mixed_entry_bytes() == g["mixed_entry"]
    assert CB.per_token_layer_bytes("hca") == g["hca_per_token_layer"]
    assert CB.per_token_layer_bytes("csa") == g["csa_per_token_layer"]
    assert round(CB.layer_bytes_at("hca") / 1e6, 1) == g["hca_layer_1m_MB"]
    assert round(CB.layer_bytes_at("csa") / 1e6) == g["csa_layer_1m_MB"]
    assert CB.window_bytes_per_layer() == g["window_per_layer"]
    pro, fl = CB.model_cache_bytes("pro"), CB.model_cache_bytes("flash")
    assert round(pro["total"] / 1e9, 2) == g["pro_total_GB"]
    assert round(pro["csa"] / 1e9, 2) == g["pro_csa_GB"]
    assert round(pro["hca"] / 1e9, 3) == g["pro_hca_GB"]
    assert round(pro["window"] / 1e6, 1) == g["pro_window_MB"]
    assert round(fl["total"] / 1e9, 2) == g["flash_total_GB"]
    assert round(fl["csa"] / 1e9, 2) == g["flash_csa_GB"]
    assert round(fl["hca"] / 1e9, 3) == g["flash_hca_GB"]
    assert round(fl["window"] / 1e6, 1) == g["flash_window_MB"]
    v32 = CB.v32_cache_bytes()
    assert round(v32 / 1e9, 1) == g["v32_total_GB"]  # 61 layers * 788 B * 2**20 tokens
    assert round(CB.gqa8_cache_bytes() / 1e9) == g["gqa8_total_GB"]
    assert round(100 * pro["total"] / CB.gqa8_cache_bytes(), 1) == g["gqa8_share_pct"]
    assert round(100 * pro["total"] / v32) == g["pro_share_pct"]
    assert round(100 * fl["total"] / v32) == g["flash_share_pct"]
    assert (1 << 20) // 4 == g["entries_1m"]
    assert round(100 * CB.share_read("pro"), 2) == g["read_share_pro_pct"]
    assert round(100 * CB.share_read("flash"), 2) == g["read_share_flash_pct"]


def test_work_per_query(golden):
    g = golden["macs_per_query"]
    assert round(CB.macs_per_query("csa_attention") / 1e6) == g["csa_attention_M"]
    assert round(CB.macs_per_query("indexer") / 1e9, 1) == g["indexer_B"]
    assert round(CB.macs_per_query("hca_attention") / 1e9, 1) == g["hca_attention_B"]
