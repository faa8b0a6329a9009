"""Compressor parity against the oracle (GPU): bulk calls, token-by-token
decode calls and chunked calls all match the oracle's entries and slot state.
Quantized entries are compared after decoding, within one quantization step
of the element's group (a float32 result may straddle a rounding boundary
that the float64 one does not)."""

import numpy as np
import pytest
import torch

from kv_cache_decode_csa_amd import _lib, synth
from oracle import codec, compressor, rope

from gpu_util import bf16, close_f32, f32, i32, need_gpu, rope_tables, say, step_bound, to_np

pytestmark = pytest.mark.gpu
ROPE_ROWS = 1 << 16


class GpuCompressor:
    """Device state + weights for one compressor; calls csa_compress."""

    def __init__(self, B, dim, ratio, d, rotate, wkv, wg, ape, fmt, entry_fmt, n_entries, tables,
                 state=None):
        self.B, self.dim, self.ratio, self.d, self.rotate = B, dim, ratio, d, rotate
        self.fmt, self.entry_fmt, self.cap = fmt, entry_fmt, n_entries
        up = bf16 if fmt == "bf16" else f32
        self.wkv, self.wg = up(wkv), up(wg)
        self.ape = f32(ape)
        self.norm = f32(np.ones(d, np.float32))
        co = 2 if ratio == 4 else 1
        shape = (B, co * ratio, co * d)
        if state is None:
            self.kv = torch.zeros(shape, dtype=torch.float32, device="cuda")
            self.sc = torch.full(shape, float("-inf"), dtype=torch.float32, device="cuda")
        else:
            self.kv, self.sc = f32(state[0]), f32(state[1])
        rb = _lib.kv_row_bytes(entry_fmt, d)
        self.entries = torch.zeros((B, n_entries, rb), dtype=torch.uint8, device="cuda")
        self.cos, self.sin = tables

    def __call__(self, x, start):
        B, T = x.shape[0], x.shape[1]
        xd = (bf16 if self.fmt == "bf16" else f32)(x)
        sp = i32(np.asarray(start, np.int32).reshape(B))
        a = _lib.make_compress_args(
            B=B, T=T, dim=self.dim, ratio=self.ratio, head_dim=self.d, rotate=self.rotate, x=xd,
            x_fmt=self.fmt, w_kv=self.wkv, w_gate=self.wg, w_fmt=self.fmt, ape=self.ape,
            norm_w=self.norm, eps=1e-6, rope_cos=self.cos, rope_sin=self.sin, start_pos=sp,
            kv_state=self.kv, score_state=self.sc, entries=self.entries, entry_fmt=self.entry_fmt,
            entries_cap=self.cap)
        ws = _lib.workspace(_lib.csa_compress_workspace_size(a))
        _lib.csa_compress(a, ws)
        torch.cuda.synchronize()

    def entry_values(self):
        e = self.entries.cpu().numpy()
        if self.entry_fmt == "f32":
            return e.view(np.float32).astype(np.float64)
        if self.entry_fmt == "bf16":
            return codec.bf16_bits_to_f64(e.view(np.uint16))
        return codec.load(e, self.entry_fmt, self.d)


def weights(rng, dim, d, ratio, scale=0.02):
    co = 2 if ratio == 4 else 1
    return ((rng.standard_normal((co * d, dim)) * scale).astype(np.float32),
            (rng.standard_normal((co * d, dim)) * scale).astype(np.float32),
            (rng.standard_normal((ratio, co * d)) * scale).astype(np.float32))


@pytest.fixture(scope="module")
def tables():
    need_gpu()
    return rope_tables(ROPE_ROWS, yarn=False)


OM = rope.frequencies(160000.0)


@pytest.mark.parametrize("ratio,d,rotate", [(4, 512, 0), (4, 128, 1), (128, 512, 0), (1, 512, 0),
                                            (2, 512, 0), (2, 128, 1)])
def test_bulk_f32(tables, ratio, d, rotate):
    B, dim, T = 2, 256, 700
    rng = np.random.default_rng(ratio * 10 + d)
    wkv, wg, ape = weights(rng, dim, d, ratio)
    x = rng.standard_normal((B, T, dim)).astype(np.float32)
    n = T // ratio + 2
    g = GpuCompressor(B, dim, ratio, d, rotate, wkv, wg, ape, "f32", "f32", n, tables)
    starts = [0, 0]
    say(f"compress bulk r={ratio} d={d}")
    g(x, starts)
    got = g.entry_values()
    for b in range(B):
        ref, st = compressor.compress_bulk(x[b].astype(np.float64), 0, wkv, wg, ape, np.ones(d),
                                           OM, ratio, d, rotate=bool(rotate))
        for i, v in ref.items():
            close_f32(got[b, i], v, tol=2e-5)
        close_f32(to_np(g.kv)[b], st[0], tol=2e-5)
        sc = to_np(g.sc)[b]
        assert np.array_equal(np.isinf(sc), np.isinf(st[1]))
        fin = np.isfinite(st[1])
        close_f32(sc[fin], st[1][fin], tol=2e-5)


@pytest.mark.parametrize("ratio,d,rotate,entry_fmt", [(4, 512, 0, "bf16"), (4, 128, 1, "bf16"),
                                                      (128, 512, 0, "fp8_mx32"),
                                                      (4, 512, 0, "mix576")])
def test_bulk_bf16_tiled_projection(tables, ratio, d, rotate, entry_fmt):
    """Many-token bf16 calls (more than 64 rows) use the tiled MFMA
    projection: 2 x 333 tokens (a ragged last 128-row tile), then a second
    call that continues from the state."""
    B, dim, T1, T2 = 2, 512, 333, 270
    rng = np.random.default_rng(7 * ratio + d)
    wkv, wg, ape = weights(rng, dim, d, ratio)
    wkv, wg = synth.bf16_round(wkv), synth.bf16_round(wg)
    x = synth.bf16_round(rng.standard_normal((B, T1 + T2, dim)).astype(np.float32))
    n = (T1 + T2) // ratio + 1
    g = GpuCompressor(B, dim, ratio, d, rotate, wkv, wg, ape, "bf16", entry_fmt, n, tables)
    say(f"compress bulk bf16 r={ratio} d={d}")
    g(x[:, :T1], [0, 0])
    g(x[:, T1:], [T1, T1])
    got = g.entry_values()
    for b in range(B):
        ref, st = compressor.compress_bulk(x[b].astype(np.float64), 0, wkv, wg, ape, np.ones(d),
                                           OM, ratio, d, rotate=bool(rotate))
        assert len(ref) == (T1 + T2) // ratio
        for i, v in ref.items():
            err = np.abs(got[b, i] - codec.store(v, entry_fmt)[1])
            assert np.all(err <= step_bound(v, entry_fmt, d)), (b, i, err.max())
        close_f32(to_np(g.kv)[b], st[0], tol=1e-4)
        sc = to_np(g.sc)[b]
        assert np.array_equal(np.isinf(sc), np.isinf(st[1]))
        fin = np.isfinite(st[1])
        close_f32(sc[fin], st[1][fin], tol=1e-4)


@pytest.mark.parametrize("entry_fmt,dim,d,rotate,ratio", [
    ("bf16", 512, 512, 0, 4), ("fp8_mx32", 512, 512, 0, 4), ("fp4_e4m3_16", 512, 512, 0, 4),
    ("f32", 512, 512, 0, 4), ("fp8_mx32", 4096, 512, 0, 4), ("fp8_mx32", 4096, 128, 1, 4),
    ("bf16", 4096, 128, 1, 4), ("fp4_mx32", 4096, 128, 1, 4),
    ("fp4_e4m3_16", 4096, 512, 0, 2), ("fp8_mx32", 4096, 128, 1, 2),
    ("fp4_e4m3_16", 4096, 512, 0, 1), ("mix576", 4096, 512, 0, 4), ("mix576", 512, 512, 0, 2)])
def test_decode_steps_bf16(tables, entry_fmt, dim, d, rotate, ratio):
    """Token-by-token calls from a state built by an earlier chunked call; each
    sequence sits at a different offset inside its block.  dim 4096 runs the
    K-sliced MFMA projection.  Ratios 2 and 1 are the CSA2 compressor of the
    V4.1-Flash diagram (no overlap; slot bias zero)."""
    B = 3
    rng = np.random.default_rng(7)
    wkv, wg, ape = (synth.bf16_round(w) for w in weights(rng, dim, d, ratio))
    ape = weights(rng, dim, d, ratio)[2] if ratio == 4 else np.zeros_like(ape)
    prefix = np.array([37, 40, 42])
    steps = 9
    x = synth.bf16_round(rng.standard_normal((B, 60, dim)).astype(np.float32))
    cap = 60 // ratio + 2
    g = GpuCompressor(B, dim, ratio, d, rotate, wkv, wg, ape, "bf16", entry_fmt, cap, tables)
    # prefix: one chunked call per sequence (different lengths -> separate calls)
    for b in range(B):
        gb = GpuCompressor(1, dim, ratio, d, rotate, wkv, wg, ape, "bf16", entry_fmt, cap, tables)
        gb(x[b:b + 1, :prefix[b]], [0])
        g.kv[b], g.sc[b], g.entries[b] = gb.kv[0], gb.sc[0], gb.entries[0]
    for s in range(steps):
        g(x[np.arange(B), prefix + s][:, None, :], prefix + s)
    got = g.entry_values()
    for b in range(B):
        T = prefix[b] + steps
        ref, st = compressor.compress_stream(x[b, :T].astype(np.float64), 0, wkv, wg, ape,
                                             np.ones(d), OM, ratio, d, rotate=bool(rotate))
        for i, v in ref.items():
            stored = codec.store(v, entry_fmt)[1]
            err = np.abs(got[b, i] - stored)
            assert np.all(err <= step_bound(v, entry_fmt, d)), (b, i, err.max())
        close_f32(to_np(g.kv)[b], st[0], tol=1e-4)


def test_hca_chunked_calls(tables):
    B, dim, d, ratio = 1, 256, 512, 128
    rng = np.random.default_rng(8)
    wkv, wg, ape = weights(rng, dim, d, ratio)
    x = rng.standard_normal((B, 420, dim)).astype(np.float32)
    g = GpuCompressor(B, dim, ratio, d, 0, wkv, wg, ape, "f32", "f32", 8, tables)
    p = 0
    for c in (100, 50, 1, 150, 119):   # completes blocks 0, 1, 2 across calls
        g(x[:, p:p + c], [p])
        p += c
    ref, st = compressor.compress_stream(x[0].astype(np.float64), 0, wkv, wg, ape, np.ones(d), OM,
                                         ratio, d)
    assert sorted(ref) == [0, 1, 2]
    got = g.entry_values()
    for i, v in ref.items():
        close_f32(got[0, i], v, tol=2e-5)
    close_f32(to_np(g.kv)[0], st[0], tol=2e-5)


def test_compress_many_equals_separate_calls(tables):
    """csa_compress_many (the main-KV and index-key compressors of a layer on
    the same token, fused) leaves exactly the entries and state that separate
    csa_compress calls leave, over steps that complete blocks."""
    B, dim, ratio = 3, 512, 4
    rng = np.random.default_rng(11)
    specs = [(512, 0, "fp8_mx32"), (128, 1, "fp8_mx32")]
    ws_ = [tuple(synth.bf16_round(w) for w in weights(rng, dim, d, ratio)) for d, _, _ in specs]
    x = synth.bf16_round(rng.standard_normal((B, 12, dim)).astype(np.float32))
    start = np.array([40, 41, 42], np.int32)
    sides = []
    for _ in range(2):
        sides.append([GpuCompressor(B, dim, ratio, d, rot, w[0], w[1], w[2], "bf16", fmt, 32, tables)
                      for (d, rot, fmt), w in zip(specs, ws_)])
    fused, sep = sides
    for s in range(9):
        pos = start + s
        xs = x[:, s:s + 1]
        for g in sep:
            g(xs, pos)
        sp = i32(pos)
        xd = bf16(xs)
        args = [_lib.make_compress_args(
            B=B, T=1, dim=dim, ratio=ratio, head_dim=g.d, rotate=g.rotate, x=xd, x_fmt="bf16",
            w_kv=g.wkv, w_gate=g.wg, w_fmt="bf16", ape=g.ape, norm_w=g.norm, eps=1e-6,
            rope_cos=g.cos, rope_sin=g.sin, start_pos=sp, kv_state=g.kv, score_state=g.sc,
            entries=g.entries, entry_fmt=g.entry_fmt, entries_cap=g.cap) for g in fused]
        ws = _lib.workspace(_lib.csa_compress_many_workspace_size(args))
        _lib.csa_compress_many(args, ws)
        torch.cuda.synchronize()
    for gf, gs in zip(fused, sep):
        assert torch.equal(gf.entries, gs.entries)
        assert torch.equal(gf.kv, gs.kv)
        assert torch.equal(gf.sc, gs.sc)


@pytest.mark.parametrize("ratio,d,rotate,efmt", [(4, 512, 0, "fp8_mx32"), (4, 128, 1, "fp8_mx32"),
                                                (128, 512, 0, "bf16")])
def test_decode_large_batch_equals_sub_batches(tables, ratio, d, rotate, efmt):
    """Single-token calls for 130 sequences (the projection then spans three
    64-row blocks) leave exactly the entries and slot state that the same
    sequences leave in calls of 10, over steps that complete blocks: a
    sequence's result does not depend on its batch."""
    B, sub, dim = 130, 10, 512
    rng = np.random.default_rng(ratio * 1000 + d)
    wkv, wg, ape = (synth.bf16_round(w) for w in weights(rng, dim, d, ratio))
    base = 40 if ratio == 4 else 120
    start = (base + rng.integers(0, 2 * ratio if ratio == 4 else 12, size=B)).astype(np.int32)
    cap = 32 if ratio == 4 else 4
    big = GpuCompressor(B, dim, ratio, d, rotate, wkv, wg, ape, "bf16", efmt, cap, tables)
    smalls = [GpuCompressor(min(sub, B - b0), dim, ratio, d, rotate, wkv, wg, ape, "bf16", efmt,
                            cap, tables) for b0 in range(0, B, sub)]
    say(f"compress large batch ratio={ratio} d={d} {efmt}: B={B} against calls of {sub}")
    for step in range(6):
        x = synth.bf16_round(rng.standard_normal((B, 1, dim)).astype(np.float32))
        pos = start + step
        big(x, pos)
        for i, g in enumerate(smalls):
            g(x[i * sub:i * sub + g.B], pos[i * sub:i * sub + g.B])
    done = 0
    for i, g in enumerate(smalls):
        b0, b1 = i * sub, i * sub + g.B
        assert torch.equal(big.entries[b0:b1], g.entries), i
        assert torch.equal(big.kv[b0:b1], g.kv), i
        assert torch.equal(big.sc[b0:b1].view(torch.int32), g.sc.view(torch.int32)), i
        done += int((g.entries != 0).any(dim=2).sum())
    assert done > 0  # some blocks completed


@pytest.mark.parametrize("entry_fmt", ["bf16", "fp8_mx32"])
def test_hca_decode_steps_bf16(tables, entry_fmt):
    """Single-token calls of the 128-token compressor across block boundaries
    (slot writes without emission, then the emitting token), each sequence at
    its own offset, against the oracle's streaming state machine."""
    B, dim, d, ratio = 2, 256, 512, 128
    rng = np.random.default_rng(12)
    wkv, wg, ape = (synth.bf16_round(w) for w in weights(rng, dim, d, ratio))
    ape = weights(rng, dim, d, ratio)[2]
    prefix = np.array([120, 250])
    steps = 12
    x = synth.bf16_round(rng.standard_normal((B, 270, dim)).astype(np.float32))
    g = GpuCompressor(B, dim, ratio, d, 0, wkv, wg, ape, "bf16", entry_fmt, 4, tables)
    for b in range(B):
        gb = GpuCompressor(1, dim, ratio, d, 0, wkv, wg, ape, "bf16", entry_fmt, 4, tables)
        gb(x[b:b + 1, :prefix[b]], [0])
        g.kv[b], g.sc[b], g.entries[b] = gb.kv[0], gb.sc[0], gb.entries[0]
    for s in range(steps):
        g(x[np.arange(B), prefix + s][:, None, :], prefix + s)
    got = g.entry_values()
    for b in range(B):
        T = prefix[b] + steps
        ref, st = compressor.compress_stream(x[b, :T].astype(np.float64), 0, wkv, wg, ape,
                                             np.ones(d), OM, ratio, d)
        assert sorted(ref) == list(range(T // ratio))
        for i, v in ref.items():
            stored = codec.store(v, entry_fmt)[1]
            err = np.abs(got[b, i] - stored)
            assert np.all(err <= step_bound(v, entry_fmt, d)), (b, i, err.max())
        close_f32(to_np(g.kv)[b], st[0], tol=1e-4)
        sc = to_np(g.sc)[b]
        assert np.array_equal(np.isinf(sc), np.isinf(st[1]))
        fin = np.isfinite(st[1])
        close_f32(sc[fin], st[1][fin], tol=1e-4)
