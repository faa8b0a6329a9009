"""Seeded synthetic inputs for the benchmark workloads.

This module holds data recipes only (shapes, seeds, value distributions and
the float32 -> bf16 cast of generated values); it contains none of the
method's arithmetic and imports nothing from the library or the oracle.
Both the GPU path and the oracle draw their inputs from here.

Every tensor has its own stream, keyed by (seed, tensor id, leading index), so
one sequence of a batch can be regenerated on its own:
``np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, b])))``.
Seeds are 20261200 + workload number.
"""

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20261200

# fixed tensor ids
T_X, T_WKV, T_WGATE, T_APE = 1, 2, 3, 4
T_IWKV, T_IWGATE, T_IAPE = 5, 6, 7
T_WINDOW, T_Q, T_QIDX, T_WIDX, T_SINK = 8, 9, 10, 11, 12
T_ENTRIES, T_IKEYS, T_XTAIL, T_TOPK, T_SCORES = 13, 14, 15, 16, 17
T_WQA, T_QNORM, T_WQB, T_WKVWIN, T_KVNORM, T_WQBI, T_WPROJ, T_WOA, T_WOB, T_O = range(20, 30)
T_RQ, T_RSINK, T_RWIN = 30, 31, 32


@dataclass
class Workload:
    """Shape and distribution recipe of one decode workload."""
    num: int
    name: str
    B: int
    ctx: int                  # tokens of context; the query sits at t = ctx - 1
    ratio: int                # 4 (CSA) or 128 (HCA)
    n_entries: int            # compressed entries per sequence = ctx // ratio
    H: int = 64               # query heads (dim 512)
    Hi: int = 64              # indexer heads (dim 128)
    topk: int = 512
    dim: int = 4096           # hidden size feeding the compressor
    theta: float = 160000.0
    yarn: bool = True
    q_fmt: str = "bf16"       # storage of q / q_idx / outputs
    ent_fmt: str = "bf16"     # main KV rows
    win_fmt: str = "bf16"     # window rows
    key_fmt: str = "bf16"     # index keys
    kv_std: float = 1.0       # std of entries / window / q
    ikey_std: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def t(self):
        return self.ctx - 1

    @property
    def seed(self):
        return SEED_BASE + self.num


WORKLOADS = {
    # tiny whole path from hidden states, fp32
    1: Workload(1, "csa_tiny_f32", B=1, ctx=2048, ratio=4, n_entries=512, H=16, Hi=4, topk=64,
                dim=1024, yarn=False, q_fmt="f32", ent_fmt="f32", win_fmt="f32", key_fmt="f32"),
    # CSA decode, bf16, 64K context, V4-Flash shape with 32 indexer heads
    2: Workload(2, "csa_64k_bf16", B=32, ctx=65536, ratio=4, n_entries=16384, H=64, Hi=32,
                topk=512, kv_std=512 ** -0.5),
    # HCA decode, bf16, 1M context
    3: Workload(3, "hca_1m_bf16", B=16, ctx=1048576, ratio=128, n_entries=8192, H=64, Hi=0,
                topk=0),
    # chunked prefill: 32768 new tokens on a 262144-token prefix
    4: Workload(4, "csa_prefill_32k_bf16", B=1, ctx=262144 + 32768, ratio=4,
                n_entries=(262144 + 32768) // 4, H=64, Hi=64, topk=512,
                extra={"prefix": 262144, "new": 32768}),
    # quantized CSA decode at 1M: FP8-528 main KV and window, FP8-132 index keys
    5: Workload(5, "csa_1m_fp8", B=8, ctx=1048576, ratio=4, n_entries=262144, H=64, Hi=64,
                topk=512, ent_fmt="fp8_mx32", win_fmt="fp8_mx32", key_fmt="fp8_mx32"),
    # V4.1-style CSA2 decoder layer group at m = 1: one entry per token (256K
    # context = 262,144 entries, the headline's entry count), MXFP4-288 main KV,
    # MXFP4-68 index keys with bf16 scores, FP8 window; one Full layer
    # (compress, index, attend) and 5 Reuse layers that attend with their own
    # queries and windows over the Full layer's entries and top-512 ids
    6: Workload(6, "csa2_m1_256k", B=8, ctx=262144, ratio=1, n_entries=262144, H=64, Hi=64,
                topk=512, ent_fmt="fp4_e4m3_16", win_fmt="fp8_mx32", key_fmt="fp4_mx32",
                extra={"csa2": True, "reuse": 5}),
}


def layer_variant(w):
    """The workload-5 variant that also runs the layer's steps on either side
    of the path: query path, index-query preparation and window-entry write
    from the token's hidden state, and the grouped output projection (V4-Flash
    shapes: q_rank 1024, 8 groups of 8 heads, o_rank 1024)."""
    import dataclasses
    return dataclasses.replace(w, name="csa_1m_fp8_layer",
                               extra=dict(w.extra, layer=dict(q_rank=1024, groups=8, o_rank=1024)))


def mxfp4_variant(w):
    """The workload-5 variant whose main KV rows are MXFP4 (E2M1 + E4M3/16)."""
    import dataclasses
    return dataclasses.replace(w, name="csa_1m_mxfp4", ent_fmt="fp4_e4m3_16")


def fp4_indexer_variant(w):
    """The workload-5 variant with the FP4 indexer: MXFP4-MX32 index keys (68 B),
    index queries carrying MXFP4 values, bf16 index scores."""
    import dataclasses
    return dataclasses.replace(w, name="csa_1m_fp4idx", key_fmt="fp4_mx32")


def batch_variant(w, B):
    """The same workload at another batch size (each sequence's data depends
    only on its own index, so the first sequences are the base workload's)."""
    import dataclasses
    return dataclasses.replace(w, name=f"{w.name}_b{B}", B=B)


def paged_variant(w):
    """The same workload served from a block cache ("DeepSeek-V4 deep dive"
    section 9.4): entries and index keys in a pool of blocks of one 128-token
    block's worth (32 CSA entries, 1 HCA entry), placed by a seeded random
    permutation and found through per-sequence block tables; window rings
    and compressor slots in a pool of 2B state slots, B of them in use."""
    import dataclasses
    be = 128 // w.ratio
    return dataclasses.replace(w, name=w.name + "_paged",
                               extra=dict(w.extra, paged=dict(block_entries=be, slots=2 * w.B)))


def rng(seed, tid, idx=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, idx])))


def normal(seed, tid, shape, std=1.0, idx=0):
    """float32 N(0, std^2) of the given shape from stream (seed, tid, idx)."""
    g = rng(seed, tid, idx)
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def normal_batched(seed, tid, B, shape, std=1.0, b_range=None):
    """[len(b_range), *shape]; element b comes from stream (seed, tid, b)."""
    bs = range(B) if b_range is None else b_range
    return np.stack([normal(seed, tid, shape, std, idx=b) for b in bs])


def bf16_round(x):
    """Round float32 values to the nearest bf16 (ties to even), as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def as_fmt_values(x, fmt):
    """Values of generated float32 data as stored before any method codec:
    bf16 inputs are rounded to bf16; f32 and quantized inputs stay float32
    (quantized formats are produced by each side's own codec)."""
    return bf16_round(x) if fmt == "bf16" else np.asarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------
# per-workload tensors (float32 values; bf16 tensors already rounded)
# ----------------------------------------------------------------------------

def queries(w, b_range=None):
    """q [B, H, 512] and sink [H]."""
    q = normal_batched(w.seed, T_Q, w.B, (w.H, 512), w.kv_std, b_range)
    sink = normal(w.seed, T_SINK, (w.H,))
    return as_fmt_values(q, w.q_fmt), sink


def index_queries(w, b_range=None):
    """q_idx [B, Hi, 128] and pre-scaled head weights w [B, Hi]."""
    qi = normal_batched(w.seed, T_QIDX, w.B, (w.Hi, 128), 1.0, b_range)
    wi = normal_batched(w.seed, T_WIDX, w.B, (w.Hi,), (128 * w.Hi) ** -0.5, b_range)
    return as_fmt_values(qi, w.q_fmt), wi


def window_rows(w, b_range=None):
    """Raw window ring [B, 128, 512] (stored, already-rotated form)."""
    return as_fmt_values(normal_batched(w.seed, T_WINDOW, w.B, (128, 512), w.kv_std, b_range),
                         w.win_fmt)


def entries(w, b_range=None):
    """Compressed main KV [B, N, 512] (stored form, before any codec)."""
    return as_fmt_values(normal_batched(w.seed, T_ENTRIES, w.B, (w.n_entries, 512), w.kv_std,
                                        b_range), w.ent_fmt)


def index_keys(w, b_range=None):
    """Index keys [B, N, 128] (stored form, before any codec)."""
    return as_fmt_values(normal_batched(w.seed, T_IKEYS, w.B, (w.n_entries, 128), w.ikey_std,
                                        b_range), w.key_fmt)


def reuse_layer_inputs(w, layer, b_range=None):
    """Queries [B, H, 512], sink [H] and window ring [B, 128, 512] of reuse
    layer `layer` >= 1 of a layer group; element b of each comes from stream
    (seed, tensor id, layer * 65536 + b)."""
    bs = range(w.B) if b_range is None else b_range
    q = np.stack([normal(w.seed, T_RQ, (w.H, 512), w.kv_std, idx=layer * 65536 + b) for b in bs])
    sink = normal(w.seed, T_RSINK, (w.H,), idx=layer)
    win = np.stack([normal(w.seed, T_RWIN, (128, 512), w.kv_std, idx=layer * 65536 + b)
                    for b in bs])
    return as_fmt_values(q, w.q_fmt), sink, as_fmt_values(win, w.win_fmt)


def compressor_weights(w, head_dim, ratio, indexer=False):
    """W_kv, W_gate [coff*d, dim] ~ N(0, 0.02^2), ape [r, coff*d] ~ N(0, 0.02^2),
    norm weight ones [d]."""
    coff = 2 if ratio == 4 else 1
    tids = (T_IWKV, T_IWGATE, T_IAPE) if indexer else (T_WKV, T_WGATE, T_APE)
    wkv = normal(w.seed, tids[0], (coff * head_dim, w.dim), 0.02)
    wg = normal(w.seed, tids[1], (coff * head_dim, w.dim), 0.02)
    ape = normal(w.seed, tids[2], (ratio, coff * head_dim), 0.02)
    if w.extra.get("csa2"):  # the CSA2 compressor has no slot bias
        ape = np.zeros_like(ape)
    fmt = w.q_fmt
    return as_fmt_values(wkv, fmt), as_fmt_values(wg, fmt), ape, np.ones(head_dim, np.float32)


def hidden(w, T, idx=0, tid=T_X):
    """Hidden states [T, dim] ~ N(0, 1) for sequence idx."""
    return as_fmt_values(normal(w.seed, tid, (T, w.dim), 1.0, idx=idx), w.q_fmt)


def random_topk_ids(seed, n_vis, k, n_pad=0, idx=0):
    """Distinct compressed ids < n_vis in random order, then n_pad -1 slots."""
    g = rng(seed, T_TOPK, idx)
    m = min(k - n_pad, n_vis)
    ids = g.choice(n_vis, size=m, replace=False).astype(np.int32)
    return np.concatenate([ids, np.full(k - m, -1, np.int32)])


def random_scores(seed, n, idx=0, ties=True):
    """float32 scores with planted exact ties and a signed zero."""
    g = rng(seed, T_SCORES, idx)
    s = g.standard_normal(n, dtype=np.float32)
    if ties and n >= 16:
        pick = g.choice(n, size=n // 8, replace=False)
        s[pick] = s[pick[0]]
        z = g.choice(n, size=4, replace=False)
        s[z[:2]] = np.float32(0.0)
        s[z[2:]] = np.float32(-0.0)
    return s


# ----------------------------------------------------------------------------
# chunked prefill (workload 4): one sequence, many rows per tensor.  Rows come
# in blocks of PREFILL_BLOCK, each block from its own stream (seed, tid, block),
# so a sampled query, token or cache row is regenerated without the rest.
# ----------------------------------------------------------------------------

PREFILL_BLOCK = 256


def _bf16_round_finite(x):
    """In-place bf16 RNE of finite float32 values (same result as bf16_round;
    32-bit arithmetic cannot overflow below the NaN/Inf patterns)."""
    u = x.reshape(-1).view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    u += r
    u &= np.uint32(0xFFFF0000)
    return x


def blocked_normal(seed, tid, row_shape, lo, hi, std=1.0, threads=8, bf16=False):
    """Rows [lo, hi) of a float32 N(0, std^2) tensor [*, *row_shape] whose
    block j of PREFILL_BLOCK rows is drawn from stream (seed, tid, j); with
    bf16=True each value is then rounded to the nearest bf16 (ties to even)."""
    import concurrent.futures as cf
    n = hi - lo
    out = np.empty((n,) + tuple(row_shape), dtype=np.float32)
    if n <= 0:
        return out
    B = PREFILL_BLOCK
    blocks = range(lo // B, (hi - 1) // B + 1)

    def fill(j):
        blk = normal(seed, tid, (B,) + tuple(row_shape), std, idx=j)
        if bf16:
            _bf16_round_finite(blk)
        a, b = max(lo, j * B), min(hi, (j + 1) * B)
        out[a - lo:b - lo] = blk[a - j * B:b - j * B]

    if len(blocks) == 1 or threads <= 1:
        for j in blocks:
            fill(j)
    else:
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, blocks))
    return out


def prefill_shape(w):
    """(prefix tokens P, new tokens T, existing entries N0, entries after the chunk N)."""
    P, T = w.extra["prefix"], w.extra["new"]
    return P, T, P // w.ratio, (P + T) // w.ratio


def prefill_rows(w, tid, row_shape, lo, hi, std=1.0):
    """Rows [lo, hi) of a prefill tensor in its stored values (bf16-rounded)."""
    return blocked_normal(w.seed, tid, row_shape, lo, hi, std, bf16=w.q_fmt == "bf16")


def prefill_queries(w, lo, hi):
    """q [hi - lo, H, 512] of new tokens lo .. hi-1 (query i sits at P + i)."""
    return prefill_rows(w, T_Q, (w.H, 512), lo, hi)


def prefill_index_queries(w, lo, hi):
    """q_idx [hi - lo, Hi, 128] and head weights [hi - lo, Hi] (pre-scaled)."""
    qi = prefill_rows(w, T_QIDX, (w.Hi, 128), lo, hi)
    wi = blocked_normal(w.seed, T_WIDX, (w.Hi,), lo, hi, (128 * w.Hi) ** -0.5)
    return qi, wi


def prefill_hidden(w, lo, hi):
    """Hidden states [hi - lo, dim] of new tokens lo .. hi-1."""
    return prefill_rows(w, T_X, (w.dim,), lo, hi)


def prefill_tail(w):
    """Hidden states [4, dim] of the prefix's last block (positions P-4 .. P-1)."""
    return as_fmt_values(normal(w.seed, T_XTAIL, (4, w.dim)), w.q_fmt)


def prefill_window(w, lo, hi):
    """Raw window KV rows [hi - lo, 512]; row r holds position P - 127 + r."""
    return prefill_rows(w, T_WINDOW, (512,), lo, hi)


def prefill_entries(w, lo, hi):
    """Existing compressed entries [hi - lo, 512] of the prefix (ids lo .. hi-1 < N0)."""
    return prefill_rows(w, T_ENTRIES, (512,), lo, hi)


def prefill_index_keys(w, lo, hi):
    """Existing index keys [hi - lo, 128] of the prefix."""
    return prefill_rows(w, T_IKEYS, (128,), lo, hi)


def prefill_sink(w):
    return normal(w.seed, T_SINK, (w.H,))


def layer_weights(seed, dim, q_rank, H, Hi, groups, o_rank):
    """Weights of the layer's input and output steps, as float32 arrays:
    projections [out, in] ~ N(0, 1/in) rounded to bf16; norm weights
    1 + N(0, 0.1^2) in float32.  Row block j of 256 rows of a projection
    comes from stream (seed, tensor id, j)."""
    def proj(tid, n_out, n_in):
        return blocked_normal(seed, tid, (n_in,), 0, n_out, n_in ** -0.5, bf16=True)

    gw = H // groups * 512
    out = {
        "wq_a": proj(T_WQA, q_rank, dim),
        "q_norm": 1.0 + normal(seed, T_QNORM, (q_rank,), 0.1),
        "wq_b": proj(T_WQB, H * 512, q_rank),
        "wkv": proj(T_WKVWIN, 512, dim),
        "kv_norm": 1.0 + normal(seed, T_KVNORM, (512,), 0.1),
        "wo_a": proj(T_WOA, groups * o_rank, gw).reshape(groups, o_rank, gw),
        "wo_b": proj(T_WOB, dim, groups * o_rank),
    }
    if Hi:
        out["wq_b_idx"] = proj(T_WQBI, Hi * 128, q_rank)
        out["w_proj"] = proj(T_WPROJ, Hi, dim)
    return out
