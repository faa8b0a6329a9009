"""Helpers for the GPU parity tests: uploads, the library's RoPE tables and
tolerance checks.  The oracle is called only by the tests themselves."""

import sys

import numpy as np
import pytest
import torch

from kv_cache_decode_csa_amd import _lib

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
