"""Pins of the oracle's composed paths (oracle/pipeline.py), CPU only.

* ``csa_decode_from_hidden``: with zero gates and zero slot biases the
  compressor's per-channel softmax gives equal weights, so every entry is the
  plain mean of its slots ("DeepSeek-V4 deep dive" section 4.1, the
  equal-score case of its worked example), normalised and rotated at its
  block's first position (section 4.2); with k >= the visible count the
  selection keeps every entry, so the output is one dense softmax over
  [window ; entries] with the sink in the denominator (sections 3.4 Eq. 27,
  5.3).  The expected value here is built from the mean by hand and the dense
  attention is torch's scaled_dot_product_attention on the CPU, with the sink
  as an extra key that carries zero value.
* ``layer_decode_step``: the query is rotated exactly once.  Its attention
  output equals the same torch attention fed with the page's rotated query
  (``layer.queries``, section 3.3), and feeding an already-rotated query back
  into the path (a double rotation) moves the output far outside any
  rounding tolerance.
"""

import numpy as np
import torch

from oracle import attention as A
from oracle import codec as C
from oracle import layer as L
from oracle import pipeline as P
from oracle import rope as R

OM = R.frequencies(160000.0)
SCALE = 512 ** -0.5


def _torch_sink_attention(qrot, rows, sink, scale):
    """softmax([q.c * scale ; sink]) over rows, the sink's value being zero:
    torch SDPA on float64 CPU tensors, one batch of H heads."""
    H, D = qrot.shape
    n = rows.shape[0]
    K = np.concatenate([rows, np.zeros((1, D))])              # extra key for the sink
    bias = np.zeros((H, 1, n + 1))
    bias[:, 0, n] = sink                                      # its logit is exactly sink_h
    q = torch.from_numpy(qrot[:, None, :])                    # [H, 1, D]
    k = torch.from_numpy(np.broadcast_to(K, (H, n + 1, D)).copy())
    o = torch.nn.functional.scaled_dot_product_attention(q, k, k, attn_mask=torch.from_numpy(bias),
                                                         scale=scale)
    return o[:, 0, :].numpy()


def test_decode_from_hidden_mean_pool_closed_form():
    rng = np.random.default_rng(71)
    T, dim, H, Hi = 83, 32, 4, 2              # t = 82: 20 complete blocks, 3 tokens pending
    t = T - 1
    n = (t + 1) // 4
    x = rng.standard_normal((T, dim))

    def comp(d):
        return dict(wkv=rng.standard_normal((2 * d, dim)) * 0.3, wgate=np.zeros((2 * d, dim)),
                    ape=np.zeros((4, 2 * d)), norm_w=np.ones(d))

    main, idx = comp(512), comp(128)
    q = rng.standard_normal((H, 512))
    qi = rng.standard_normal((Hi, 128))
    wi = rng.standard_normal(Hi)
    sink = rng.standard_normal(H)
    win = rng.standard_normal((128, 512))
    k = n + 5                                 # k >= visible: everything is selected
    ref = P.csa_decode_from_hidden(x, main, idx, q, qi, wi, sink, win, t, k, OM)

    # entries by hand: the mean of block i's 4 tokens (channels d..2d) and of
    # block i-1's 4 tokens (channels 0..d), block 0 without a previous block
    v = x @ main["wkv"].T
    E = np.zeros((n, 512))
    for i in range(n):
        slots = [v[4 * i + a, 512:] for a in range(4)]
        if i > 0:
            slots += [v[4 * i - 4 + a, :512] for a in range(4)]
        c = np.mean(slots, axis=0)
        c = c / np.sqrt(np.mean(c * c) + 1e-6)
        E[i] = R.rotate(c, 4 * i, OM)
    E = E.astype(np.float32).astype(np.float64)   # stored as float32 rows (the default format)
    np.testing.assert_allclose(ref["entries"], E, rtol=1e-12, atol=1e-12)
    assert sorted(ref["topk"][:n].tolist()) == list(range(n))
    assert np.all(ref["topk"][n:] == -1)

    # one dense softmax over the window (positions t-127 .. t; all >= 0 only
    # from position 0, so rows of negative positions are left out) and E
    p = np.arange(t - 127, t + 1)
    wrows = win[p[p >= 0] % 128]
    rows = np.concatenate([wrows, E])
    qrot = R.rotate(q, t, OM)
    o = _torch_sink_attention(qrot, rows, sink, SCALE)
    o = R.rotate(o, t, OM, inverse=True)
    np.testing.assert_allclose(ref["out"], o, rtol=1e-10, atol=1e-12)


def _layer_case(seed=5):
    rng = np.random.default_rng(seed)
    dim, q_rank, H, Hi, groups, o_rank = 256, 256, 16, 4, 2, 32
    wn = {
        "wq_a": rng.standard_normal((q_rank, dim)) / np.sqrt(dim),
        "q_norm": 1 + 0.1 * rng.standard_normal(q_rank),
        "wq_b": rng.standard_normal((H * 512, q_rank)) / np.sqrt(q_rank),
        "wkv": rng.standard_normal((512, dim)) / np.sqrt(dim),
        "kv_norm": 1 + 0.1 * rng.standard_normal(512),
        "wq_b_idx": rng.standard_normal((Hi * 128, q_rank)) / np.sqrt(q_rank),
        "w_proj": rng.standard_normal((Hi, dim)) / np.sqrt(dim),
        "wo_a": rng.standard_normal((groups, o_rank, H // groups * 512)) / np.sqrt(4096),
        "wo_b": rng.standard_normal((dim, groups * o_rank)) / np.sqrt(groups * o_rank),
        "H": H, "Hi": Hi,
    }
    N = 40
    t = 4 * N + 37                            # all 40 entries visible, ring full
    x = rng.standard_normal(dim)
    ring = rng.standard_normal((128, 512))
    E = rng.standard_normal((N, 512))
    K = rng.standard_normal((N, 128))
    sink = rng.standard_normal(H)
    return wn, x, t, ring, E, K, sink


def test_layer_step_rotates_query_once():
    wn, x, t, ring, E, K, sink = _layer_case()
    step = P.layer_decode_step(x, t, wn, ring, "f32", E, K, sink, 64, OM)
    # the window entry lands in slot t mod 128, stored in the ring's format
    assert np.array_equal(step["ring"][t % 128], C.store(step["kv"], "f32")[1])
    others = np.arange(128) != t % 128
    assert np.array_equal(step["ring"][others], ring[others])
    # every entry is visible and k > N: all are selected
    assert sorted(step["topk"][:40].tolist()) == list(range(40))
    # the page's query (rotated once at t) against the rows as stored
    qr = L.latent(x, wn["wq_a"], wn["q_norm"])
    q_page = L.queries(qr, wn["wq_b"], wn["H"], t, OM)
    rows = np.concatenate([step["ring"][A.window_ids(t)], E])
    o = R.rotate(_torch_sink_attention(q_page, rows, sink, SCALE), t, OM, inverse=True)
    np.testing.assert_allclose(step["out"], o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(step["y"], L.output_projection(o, wn["wo_a"], wn["wo_b"]),
                               rtol=1e-9, atol=1e-12)
    # a query rotated twice breaks the relative-position property: the output
    # moves by far more than bf16 rounding could
    o2 = A.sparse_decode(q_page, step["ring"], A.window_ids(t), E, step["topk"], sink, SCALE, t,
                         OM)
    rel = np.abs(o2 - o).max() / np.abs(o).max()
    assert rel > 0.05, rel


def test_layer_step_given_ids_permutation():
    """Attending over a given list equals the oracle's own selection when the
    list is a permutation of it (section 3.4: one softmax over a set)."""
    wn, x, t, ring, E, K, sink = _layer_case(6)
    a = P.layer_decode_step(x, t, wn, ring, "bf16", E, K, sink, 16, OM)
    ids = a["topk"][::-1].copy()
    b = P.layer_decode_step(x, t, wn, ring, "bf16", E, K, sink, 16, OM, ids=ids)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-14)
    assert len(set(a["topk"].tolist())) == 16
