"""Pins for the oracle's compressor (CPU only)."""

import math

import numpy as np
import pytest

from oracle import compressor as C
from oracle import rope


def _params(rng, dim, d, ratio):
    co = C.coff_of(ratio)
    return dict(w_kv=rng.standard_normal((co * d, dim)) * 0.3,
                w_gate=rng.standard_normal((co * d, dim)) * 0.3,
                ape=rng.standard_normal((ratio, co * d)) * 0.3,
                norm_w=1.0 + 0.1 * rng.standard_normal(d))


OM = rope.frequencies(160000.0, rope.V4_YARN)


def test_pool_worked_example(golden):
    g = golden["pooling"]
    v = np.array(g["values"], dtype=float)[:, None]
    s = np.array([0, 0, 0, math.log(5)])[:, None]
    assert abs(C._pool(v, s)[0] - g["entry_peaked"]) < 1e-12
    w = np.exp(s[:, 0]) / np.exp(s[:, 0]).sum()
    np.testing.assert_allclose(w, g["weights_peaked"], atol=1e-12)
    assert abs(C._pool(v, np.ones((4, 1)))[0] - g["entry_equal"]) < 1e-12


def test_prompt10(golden):
    g = golden["compressor_prompt10"]
    rng = np.random.default_rng(0)
    dim, d = 8, 64
    P = _params(rng, dim, d, 4)
    x = rng.standard_normal((g["tokens"], dim))
    out, _ = C.compress_stream(x, 0, P["w_kv"], P["w_gate"], P["ape"], P["norm_w"], OM, 4, d)
    assert sorted(out) == g["csa_entries"]
    # entry 1 pools tokens 0..7: perturbing token 0 or 7 changes it, 8/9 do not exist yet
    for tok, changes in ((0, True), (7, True)):
        x2 = x.copy()
        x2[tok] += 1.0
        o2, _ = C.compress_stream(x2, 0, P["w_kv"], P["w_gate"], P["ape"], P["norm_w"], OM, 4, d)
        assert (np.max(np.abs(o2[1] - out[1])) > 1e-6) == changes
    # entry 0 does not read token 4
    x3 = x.copy()
    x3[4] += 1.0
    o3, _ = C.compress_stream(x3, 0, P["w_kv"], P["w_gate"], P["ape"], P["norm_w"], OM, 4, d)
    np.testing.assert_array_equal(o3[0], out[0])
    # RoPE positions 0 and 4: rotating back by those positions gives the un-rotated norm
    for i, p in zip(g["csa_entries"], g["csa_rope_pos"]):
        assert p == i * 4
    # HCA: nothing yet
    P128 = _params(rng, dim, d, 128)
    o128, _ = C.compress_stream(x, 0, P128["w_kv"], P128["w_gate"], P128["ape"],
                                P128["norm_w"], OM, 128, d)
    assert len(o128) == g["hca_entries"]


def test_prompt1000(golden):
    g = golden["compressor_prompt1000"]
    rng = np.random.default_rng(1)
    dim, d = 4, 64
    x = rng.standard_normal((g["tokens"], dim))
    P = _params(rng, dim, d, 4)
    out, (kv, sc) = C.compress_bulk(x, 0, P["w_kv"], P["w_gate"], P["ape"], P["norm_w"], OM, 4, d)
    assert len(out) == g["csa_entries"] == max(out) + 1
    lo, hi = g["csa_state_tokens"]
    v, s = C.project(x[lo:hi + 1], P["w_kv"], P["w_gate"], P["ape"], np.arange(lo, hi + 1), 4)
    np.testing.assert_allclose(kv[:4], v, atol=1e-12)  # previous slots: block 249
    np.testing.assert_allclose(sc[:4], s, atol=1e-12)
    P = _params(rng, dim, d, 128)
    out, (kv, sc) = C.compress_bulk(x, 0, P["w_kv"], P["w_gate"], P["ape"], P["norm_w"], OM,
                                    128, d)
    assert len(out) == g["hca_entries"] and max(out) == 6
    assert (max(out) + 1) * 128 - 1 == g["hca_covered_last"]
    lo, hi = g["hca_tail"]
    assert hi - lo + 1 == g["hca_tail_len"]
    v, s = C.project(x[lo:hi + 1], P["w_kv"], P["w_gate"], P["ape"], np.arange(lo, hi + 1), 128)
    np.testing.assert_allclose(kv[:g["hca_tail_len"]], v, atol=1e-12)
    np.testing.assert_allclose(sc[:g["hca_tail_len"]], s, atol=1e-12)


@pytest.mark.parametrize("ratio,d,rotate", [(4, 64, False), (4, 128, True), (128, 64, False),
                                            (1, 64, False), (2, 64, False), (2, 128, True)])
def test_stream_equals_bulk_any_chunking(ratio, d, rotate):
    rng = np.random.default_rng(2 + ratio)
    dim = 16
    T = 700 if ratio == 128 else 61
    P = _params(rng, dim, d, ratio)
    x = rng.standard_normal((T, dim))
    args = (P["w_kv"], P["w_gate"], P["ape"], P["norm_w"], OM, ratio, d)
    ref, st_ref = C.compress_stream(x, 0, *args, rotate=rotate)
    for cuts in ([T], [1] * 5 + [T - 5], [3, 7, 1, 13, T - 24], [T - 1, 1]):
        st = None
        got = {}
        p = 0
        for c in cuts:
            o, st = C.compress_bulk(x[p:p + c], p, *args, rotate=rotate, state=st)
            got.update(o)
            p += c
        assert sorted(got) == sorted(ref)
        for i in ref:
            np.testing.assert_allclose(got[i], ref[i], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(st[0], st_ref[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(np.isinf(st[1]), np.isinf(st_ref[1]))
        fin = np.isfinite(st_ref[1])
        np.testing.assert_allclose(st[1][fin], st_ref[1][fin], rtol=1e-12, atol=1e-12)


def test_ratio1_closed_form():
    rng = np.random.default_rng(9)
    dim, d = 8, 64
    P = _params(rng, dim, d, 1)
    x = rng.standard_normal((5, dim))
    out, _ = C.compress_bulk(x, 3, P["w_kv"], P["w_gate"], P["ape"], P["norm_w"], OM, 1, d)
    for j in range(5):
        v = P["w_kv"] @ x[j]
        y = v / np.sqrt(np.mean(v * v) + 1e-6) * P["norm_w"]
        y = rope.rotate(y, 3 + j, OM)
        np.testing.assert_allclose(out[3 + j], y, rtol=1e-12, atol=1e-12)


def test_equal_gates_give_mean_pooling():
    rng = np.random.default_rng(10)
    dim, d = 8, 64
    P = _params(rng, dim, d, 4)
    wg = np.zeros_like(P["w_gate"])
    ape = np.zeros_like(P["ape"])
    x = rng.standard_normal((12, dim))
    out, _ = C.compress_bulk(x, 0, P["w_kv"], wg, ape, P["norm_w"], OM, 4, d)
    V = x @ P["w_kv"].T
    for i in range(3):
        cur = V[4 * i:4 * i + 4, d:]
        slots = cur if i == 0 else np.concatenate([V[4 * i - 4:4 * i, :d], cur])
        m = slots.mean(axis=0)
        y = m / np.sqrt(np.mean(m * m) + 1e-6) * P["norm_w"]
        np.testing.assert_allclose(out[i], rope.rotate(y, 4 * i, OM), rtol=1e-12, atol=1e-12)


def test_hadamard_orthogonal():
    H = C.hadamard(128)
    np.testing.assert_array_equal(H @ H.T, 128 * np.eye(128))
    assert set(np.unique(H)) == {-1.0, 1.0}


def test_ratio2_without_overlap_or_bias():
    """The V4.1 CSA2 compressor at m = 2 (V4.1-Flash diagram: encoder layers):
    no overlap and zero slot bias, so entry i pools exactly tokens 2i, 2i+1
    with a per-channel softmax of their gate scores -- with equal gates their
    mean -- then RMSNorm and RoPE at position 2i."""
    rng = np.random.default_rng(12)
    dim, d = 8, 64
    P = _params(rng, dim, d, 2)
    assert P["w_kv"].shape == (d, dim)  # coff 1: no doubled projection
    x = rng.standard_normal((9, dim))
    zero = np.zeros((2, d))
    out, st = C.compress_bulk(x, 0, P["w_kv"], P["w_gate"], zero, P["norm_w"], OM, 2, d)
    assert sorted(out) == [0, 1, 2, 3]
    V, S = x @ P["w_kv"].T, x @ P["w_gate"].T
    for i in range(4):
        e = np.exp(S[2 * i:2 * i + 2] - S[2 * i:2 * i + 2].max(axis=0))
        pooled = (e * V[2 * i:2 * i + 2]).sum(axis=0) / e.sum(axis=0)
        y = pooled / np.sqrt(np.mean(pooled ** 2) + 1e-6) * P["norm_w"]
        np.testing.assert_allclose(out[i], rope.rotate(y, 2 * i, OM), rtol=1e-12, atol=1e-12)
    # token 8 waits in slot 0 for its partner
    np.testing.assert_allclose(st[0][0], V[8], rtol=1e-12)
    eq, _ = C.compress_bulk(x, 0, P["w_kv"], np.zeros_like(P["w_gate"]), zero, P["norm_w"], OM,
                            2, d)
    m = V[0:2].mean(axis=0)
    np.testing.assert_allclose(eq[0], rope.rotate(m / np.sqrt(np.mean(m * m) + 1e-6) *
                                                  P["norm_w"], 0, OM), rtol=1e-12, atol=1e-12)
