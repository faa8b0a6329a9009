"""Pins of the oracle's layer steps around the decode path (oracle/layer.py):
the pages' parameter counts, the per-head RMS and logit ceiling, the relative
position property of the partial RoPE, the Hadamard rotation's invariance of
index scores, the index-weight scale, the ring slot, and the grouped output
projection against a dense block-diagonal one."""

import numpy as np
import pytest
from scipy.linalg import block_diag

from oracle import codec as C
from oracle import compressor as CP
from oracle import layer as L
from oracle import rope as R

OMEGA = R.frequencies(160000.0, R.V4_YARN)


def _rng(s=0):
    return np.random.default_rng(1234 + s)


@pytest.mark.parametrize("model", ["pro", "flash"])
def test_param_counts_match_pages(golden, model):
    g = golden["layer_params"][model]
    got = L.param_counts(g["dim"], g["q_rank"], g["H"], g["groups"], g["o_rank"], g.get("Hi", 0))
    for k, v in g["millions"].items():
        assert round(got[k] / 1e6, 1 if v >= 1 else 2) == v, (k, got[k])
    if "query_low_rank_millions" in g:
        assert round((got["wq_a"] + got["wq_b"]) / 1e6, 1) == g["query_low_rank_millions"]


def test_group_of_heads(golden):
    """Group 3 of Pro is heads 24..31: changing only those heads changes only
    group 3's slice of the concatenated intermediate."""
    lo, hi = golden["layer_params"]["pro_group3_heads"]
    H, g, r = 128, 16, 2
    rng = _rng(1)
    wo_a = rng.standard_normal((g, r, 8 * 512))
    wo_b = np.eye(g * r)  # identity second stage exposes the intermediate
    o = rng.standard_normal((H, 512))
    o2 = o.copy()
    o2[lo:hi + 1] += rng.standard_normal((hi - lo + 1, 512))
    d = L.output_projection(o2, wo_a, wo_b) - L.output_projection(o, wo_a, wo_b)
    changed = np.flatnonzero(np.abs(d) > 0)
    assert set(changed.tolist()) <= set(range(3 * r, 4 * r)) and len(changed) > 0


def test_output_projection_is_block_diagonal_dense():
    """The two-stage grouped projection equals one dense map by the
    block-diagonal matrix of the wo_a slices followed by wo_b."""
    rng = _rng(2)
    H, g, r, dim = 16, 2, 3, 5
    wo_a = rng.standard_normal((g, r, 8 * 512))
    wo_b = rng.standard_normal((dim, g * r))
    o = rng.standard_normal((4, H, 512))
    dense = block_diag(*[wo_a[k] for k in range(g)])  # [g r, H 512]
    mid = C.round_to_bf16(o.reshape(4, H * 512) @ dense.T)
    np.testing.assert_allclose(L.output_projection(o, wo_a, wo_b), mid @ wo_b.T, rtol=1e-12,
                               atol=1e-12)


def _weights(rng, dim=256, q_rank=128, H=4, Hi=2):
    # heads of very different scale, so a rescale across heads would show
    wq_b = rng.standard_normal((H * 512, q_rank)) * 0.05
    wq_b *= np.repeat(10.0 ** np.arange(H), 512)[:, None]
    return {
        "H": H, "Hi": Hi,
        "wq_a": rng.standard_normal((q_rank, dim)) * 0.05,
        "q_norm": 1.0 + 0.1 * rng.standard_normal(q_rank),
        "wq_b": wq_b,
        "wkv": rng.standard_normal((512, dim)) * 0.05,
        "kv_norm": np.ones(512),
        "wq_b_idx": rng.standard_normal((Hi * 128, q_rank)) * 0.05,
        "w_proj": rng.standard_normal((Hi, dim)) * 0.05,
    }


def test_query_heads_have_unit_rms_and_logit_ceiling(golden):
    """Every query head ends with RMS 1 (no learned weight) whatever its scale
    before; with unit kv_norm weights the window entry has RMS 1 too, so a
    logit q.c / sqrt(512) is at most sqrt(512) ~ 22.6 (section 3.2)."""
    g = golden["logit_ceiling"]
    rng = _rng(3)
    w = _weights(rng)
    x = rng.standard_normal((3, 256)) * 7.0
    q, _, _, kv = L.layer_input(x, np.array([5, 900, 70000]), w, OMEGA)
    rms = np.sqrt(np.mean(q * q, axis=-1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-5)
    np.testing.assert_allclose(np.sqrt(np.mean(kv * kv, axis=-1)), 1.0, rtol=1e-5)
    assert round(np.linalg.norm(q[0, 0]), 1) == g["query_length"]
    assert round(np.sqrt(512.0), 1) == g["max_logit"]
    logits = np.einsum("bhd,cd->bhc", q, kv) / np.sqrt(512.0)
    assert np.abs(logits).max() <= g["max_logit"] + 0.05
    # the ceiling is reached when the entry points along the query
    assert np.isclose(q[0, 0] @ q[0, 0], g["max_dot"], rtol=1e-5)


def test_latent_is_normalised_and_bf16():
    rng = _rng(4)
    w = _weights(rng)
    x = rng.standard_normal((2, 256))
    qr = L.latent(x, w["wq_a"], w["q_norm"])
    np.testing.assert_array_equal(qr, C.round_to_bf16(qr))
    plain = qr / w["q_norm"]
    np.testing.assert_allclose(np.sqrt(np.mean(plain ** 2, axis=-1)), 1.0, rtol=1e-2)


def test_rope_on_last_64_relative(golden):
    """Shifting the query's and the window entry's positions together leaves
    their scores unchanged (section 3.3), while the first 448 dims do not
    depend on position at all."""
    shift = golden["rope_relative"]["shift"]
    rng = _rng(5)
    w = _weights(rng)
    x = rng.standard_normal((2, 256))
    p = np.array([37, 4000])
    q1, qi1, _, _ = L.layer_input(x[0], p[0], w, OMEGA)
    q2, qi2, _, _ = L.layer_input(x[0], p[0] + shift, w, OMEGA)
    kv1 = L.window_entry(x[1], w["wkv"], w["kv_norm"], p[1], OMEGA)
    kv2 = L.window_entry(x[1], w["wkv"], w["kv_norm"], p[1] + shift, OMEGA)
    np.testing.assert_allclose(q1 @ kv1, q2 @ kv2, rtol=1e-9, atol=1e-9)
    np.testing.assert_array_equal(q1[:, :448], q2[:, :448])
    assert not np.allclose(q1[:, 448:], q2[:, 448:])
    # index queries against a key rotated the same way (RoPE then Hadamard)
    kraw = rng.standard_normal(128)
    ka = CP.postprocess(kraw, 10, 4, np.ones(128), OMEGA, True)
    kb = CP.postprocess(kraw, 10 + shift // 4, 4, np.ones(128), OMEGA, True)
    qa = L.index_queries(L.latent(x[0], w["wq_a"], w["q_norm"]), w["wq_b_idx"], 2, 100, OMEGA)
    qb = L.index_queries(L.latent(x[0], w["wq_a"], w["q_norm"]), w["wq_b_idx"], 2, 100 + shift,
                         OMEGA)
    np.testing.assert_allclose(qa @ ka, qb @ kb, rtol=1e-9, atol=1e-9)


def test_hadamard_leaves_index_scores_unchanged():
    """The rotation is orthogonal: scores of rotated queries against rotated
    keys equal those of the unrotated pair (section 5.2)."""
    rng = _rng(6)
    w = _weights(rng)
    qr = L.latent(rng.standard_normal(256), w["wq_a"], w["q_norm"])
    qi = L.index_queries(qr, w["wq_b_idx"], 2, 77, OMEGA)
    q_plain = R.rotate((qr @ w["wq_b_idx"].T).reshape(2, 128), 77, OMEGA)
    kraw = rng.standard_normal((5, 128))
    k_rot = CP.postprocess(kraw, 3, 4, np.ones(128), OMEGA, True)
    k_plain = CP.postprocess(kraw, 3, 4, np.ones(128), OMEGA, False)
    np.testing.assert_allclose(qi @ k_rot.T, q_plain @ k_plain.T, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(qi, axis=-1), np.linalg.norm(q_plain, axis=-1))
    assert not np.allclose(qi, q_plain)


def test_index_weight_scale(golden):
    """weights_proj rows that pick single channels give w_h = x_h / sqrt(128 * 64)."""
    g = golden["index_weight_scale"]
    Hi, dim = g["heads"], 256
    x = _rng(7).standard_normal(dim)
    w = L.index_weights(x, np.eye(Hi, dim))
    np.testing.assert_allclose(w, x[:Hi] / np.sqrt(g["head_dim"] * g["heads"]), rtol=1e-15)


def test_window_ring_slot():
    ring = np.zeros((128, 3))
    row = np.array([1.0, 2.0, 3.0])
    out = L.window_write(ring, row, 130)
    assert np.flatnonzero(out.any(axis=1)).tolist() == [2]
    np.testing.assert_array_equal(out[2], row)
    assert not ring.any()
    assert not L.window_write(ring, row, -1).any()
