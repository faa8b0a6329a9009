"""Helpers for the GPU parity tests: uploads, the library's RoPE tables,
tolerance checks and the selection check (which calls the oracle's top-k;
this module is test infrastructure like the oracle itself)."""

import sys

import numpy as np
import pytest
import torch

from kv_cache_decode_csa_amd import _lib
from oracle import topk as _TK

YARN = dict(factor=16.0, orig_len=65536, beta_fast=32.0, beta_slow=1.0)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()  # loud failure if the library is missing


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def bf16(x):
    """Upload float32 values that are already bf16-representable, exactly."""
    return f32(x).to(torch.bfloat16)


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def upload_rows(x, fmt):
    """float32 values [..., D] -> device rows in `fmt` (quantized by the library)."""
    if fmt == "f32":
        return f32(x)
    if fmt == "bf16":
        return bf16(x)
    D = x.shape[-1]
    rows = int(np.prod(x.shape[:-1]))
    src = f32(x)
    rb = _lib.kv_row_bytes(fmt, D)
    dst = torch.empty(x.shape[:-1] + (rb,), dtype=torch.uint8, device="cuda")
    _lib.kv_quantize(src, "f32", dst, fmt, rows, D)
    return dst


def rope_tables(rows, theta=160000.0, yarn=True):
    cos = torch.empty((rows, 32), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    if yarn:
        _lib.csa_rope_table(theta, YARN["factor"], YARN["orig_len"], YARN["beta_fast"],
                            YARN["beta_slow"], rows, cos, sin)
    else:
        _lib.csa_rope_table(theta, 0.0, 0, 0.0, 0.0, rows, cos, sin)
    return cos, sin


def close_bf16(got, ref, atol=1e-2, rtol=2e-2):
    """bf16 outputs: |g - r| <= atol + rtol |r| elementwise."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outside tolerance; "
                           f"max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")


def close_f32(got, ref, tol=1e-5):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > tol + tol * np.abs(ref)
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outside tolerance; "
                           f"max err {err.max():.3e}")


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


# ---------------------------------------------------------------- shared checks

U = 2.0 ** -24


def score_bound(q, w, K):
    """|fp32 result - exact| bound: sum_h |w_h| (130 u sum_c |q_hc k_c|) + 70 u sum_h |w_h relu_h|."""
    a = np.abs(K) @ np.abs(q).T  # [n, H]
    d = np.maximum(K @ q.T, 0)
    return 130 * U * (a @ np.abs(w)) + 70 * U * (d @ np.abs(w)) + 1e-30


def check_selection(idx, S_gpu, S_ref, tol, nv, k):
    ke = min(k, nv)
    sel = idx[:ke]
    assert np.all(idx[ke:] == -1)
    assert len(set(sel.tolist())) == ke and np.all((sel >= 0) & (sel < nv))
    # ordered by the library's own scores, ties by index
    g = S_gpu[sel]
    for a in range(ke - 1):
        assert g[a] > g[a + 1] or (g[a] == g[a + 1] and sel[a] < sel[a + 1])
    if ke < nv:
        rest = np.setdiff1d(np.arange(nv), sel)
        last = g[-1]
        assert np.all((S_gpu[rest] < last) | ((S_gpu[rest] == last) & (rest > sel[-1])))
    # against the oracle's own selection, away from near-ties
    want = _TK.topk(S_ref[:nv].astype(np.float32), k, nv)[:ke]
    diff = np.setxor1d(sel, want)
    if len(diff):
        thr = np.sort(S_ref[:nv])[::-1][ke - 1] if ke > 0 else 0
        assert np.all(np.abs(S_ref[diff] - thr) <= 2 * tol[diff] + 1e-12), diff[:10]


def step_bound(ref, fmt, d):
    """One quantization step of each element's group at the oracle's value."""
    if fmt in ("f32",):
        return 1e-5 + 1e-5 * np.abs(ref)
    if fmt == "bf16":
        return 1e-3 + 2.0 ** -7 * np.abs(ref)
    if fmt == "mix576":  # FP8 blocks of 64 on dims 0..447, bf16 on 448..511
        nope = ref[..., :448].reshape(ref.shape[:-1] + (7, 64))
        amax = np.abs(nope).max(-1, keepdims=True)
        # one E4M3 step at the element's own value (3 mantissa bits), or the
        # block's subnormal spacing
        step = np.maximum(np.abs(nope) * 2.0 ** -3, amax / 448 * 2.0 ** -3 * 2)
        step = step.reshape(ref.shape[:-1] + (448,))
        return np.concatenate([step + 1e-6, 1e-3 + 2.0 ** -7 * np.abs(ref[..., 448:])], axis=-1)
    g = 16 if fmt == "fp4_e4m3_16" else 32
    amax = np.abs(ref).reshape(ref.shape[:-1] + (d // g, g)).max(-1, keepdims=True)
    if fmt == "fp8_mx32":
        step = amax / 448 * 2.0 ** -3 * 2      # coarsest e4m3 spacing in the group, x2 margin
    elif fmt == "fp4_mx32":
        step = amax / 4 * 2.0 * 1.2            # E2M1 spacing 2 at the top, times 2**X <= amax / 4
    else:
        step = amax / 6 * 2.0 * 1.2            # coarsest e2m1 spacing (2) times the scale
    return np.broadcast_to(step, ref.shape[:-1] + (d // g, g)).reshape(ref.shape) + 1e-6
