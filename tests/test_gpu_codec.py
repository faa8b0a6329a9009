"""Codec and RoPE-table parity: the library against the oracle (GPU)."""

import numpy as np
import pytest
import torch

from kv_cache_decode_csa_amd import _lib
from oracle import codec, rope

from gpu_util import YARN, f32, need_gpu, rope_tables, say

pytestmark = pytest.mark.gpu


def _edge_rows(D, rng):
    """Rows exercising zero groups, tiny and huge values, exact e4m3 / e2m1
    midpoints, NaN and Inf."""
    rows = [rng.standard_normal(D), np.zeros(D), rng.standard_normal(D) * 1e-38,
            rng.standard_normal(D) * 3e37, rng.standard_normal(D) * 448,
            rng.uniform(-1, 1, D) * 2.0 ** rng.integers(-140, 120, D)]
    mid = np.zeros(D)
    mid[:32] = [448.0] + [(1 + (2 * k + 1) / 16) for k in range(7)] * 4 + [1e-3, 2.0 ** -9 * 2.5,
                                                                           -0.0]
    rows.append(mid)
    fp4 = np.zeros(D)
    fp4[:16] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 7.0, 0.1, -0.0, 4.5,
                2.9, 6.0]
    rows.append(fp4)
    special = rng.standard_normal(D)
    special[3] = np.nan
    special[40] = np.inf
    special[77] = -np.inf
    rows.append(special)
    return np.array(rows, dtype=np.float32)


def oracle_quantize(x, fmt):
    if fmt == "mix576":
        return codec.quantize_mix576(np.asarray(x, dtype=np.float64))
    if fmt == "fp8_mx32":
        return codec.quantize_fp8_mx32(np.asarray(x, dtype=np.float64))
    if fmt == "fp4_mx32":
        return codec.quantize_fp4_mx32(x)
    return codec.quantize_fp4_e4m3_16(x)


@pytest.mark.parametrize("D", [512, 128])
@pytest.mark.parametrize("fmt", ["fp8_mx32", "fp4_e4m3_16", "fp4_mx32"])
def test_quantize_bit_exact(D, fmt):
    need_gpu()
    rng = np.random.default_rng(11)
    x = np.concatenate([_edge_rows(D, rng), rng.standard_normal((3000, D)).astype(np.float32)])
    say(f"quantize {fmt} D={D} rows={len(x)}")
    rb = _lib.kv_row_bytes(fmt, D)
    dst = torch.empty((len(x), rb), dtype=torch.uint8, device="cuda")
    _lib.kv_quantize(f32(x), "f32", dst, fmt, len(x), D)
    got = dst.cpu().numpy()
    want = oracle_quantize(x, fmt)
    mism = np.argwhere(got != want)
    assert len(mism) == 0, f"{len(mism)} bytes differ, first {mism[:5].tolist()}"
    # bf16 input path: same bytes as quantizing the bf16 values
    xb = torch.from_numpy(x[9:]).to(torch.bfloat16).cuda()
    dst2 = torch.empty((len(x) - 9, rb), dtype=torch.uint8, device="cuda")
    _lib.kv_quantize(xb, "bf16", dst2, fmt, len(x) - 9, D)
    xv = xb.float().cpu().numpy()
    np.testing.assert_array_equal(dst2.cpu().numpy(), oracle_quantize(xv, fmt))


def test_mix576_quantize_bit_exact():
    """The V4 mixed row: device bytes equal the oracle's, from f32 and bf16 input."""
    need_gpu()
    rng = np.random.default_rng(13)
    x = np.concatenate([_edge_rows(512, rng), rng.standard_normal((2000, 512)).astype(np.float32)])
    x[-1, 448:] = np.float32(np.nan)
    say(f"quantize mix576 rows={len(x)}")
    dst = torch.empty((len(x), 592), dtype=torch.uint8, device="cuda")
    _lib.kv_quantize(f32(x), "f32", dst, "mix576", len(x), 512)
    got = dst.cpu().numpy()
    mism = np.argwhere(got != oracle_quantize(x, "mix576"))
    assert len(mism) == 0, f"{len(mism)} bytes differ, first {mism[:5].tolist()}"
    xb = torch.from_numpy(x[9:]).to(torch.bfloat16).cuda()
    dst2 = torch.empty((len(x) - 9, 592), dtype=torch.uint8, device="cuda")
    _lib.kv_quantize(xb, "bf16", dst2, "mix576", len(x) - 9, 512)
    np.testing.assert_array_equal(dst2.cpu().numpy(),
                                  oracle_quantize(xb.float().cpu().numpy(), "mix576"))
    with pytest.raises(_lib.CsaError):
        _lib.kv_quantize(f32(x[:, :128]), "f32", dst, "mix576", len(x), 128)


@pytest.mark.parametrize("fmt", ["fp8_mx32", "fp4_e4m3_16", "fp4_mx32", "mix576"])
def test_dequantize_exact(fmt):
    need_gpu()
    D = 512
    rng = np.random.default_rng(12)
    x = np.concatenate([_edge_rows(D, rng), rng.standard_normal((500, D)).astype(np.float32)])
    rows = oracle_quantize(x, fmt)
    src = torch.from_numpy(rows).cuda()
    out = torch.empty((len(x), D), dtype=torch.float32, device="cuda")
    _lib.kv_dequantize(src, fmt, out, "f32", len(x), D)
    want = codec.load(rows, fmt, D)
    got = out.cpu().numpy().astype(np.float64)
    fin = np.isfinite(want)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    # exact wherever the value is a normal float32 (subnormal products may flush)
    ok = fin & (np.abs(want) >= 2.0 ** -126) | (want == 0)
    np.testing.assert_array_equal(got[ok], want[ok])
    outb = torch.empty((len(x), D), dtype=torch.bfloat16, device="cuda")
    _lib.kv_dequantize(src, fmt, outb, "bf16", len(x), D)
    wb = codec.round_to_bf16(want.astype(np.float32))
    gb = outb.float().cpu().numpy()
    np.testing.assert_array_equal(gb[ok], wb[ok])


def test_bf16_and_f32_casts():
    need_gpu()
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((64, 256)) * 3).astype(np.float32)
    out = torch.empty((64, 256), dtype=torch.bfloat16, device="cuda")
    _lib.kv_quantize(f32(x), "f32", out, "bf16", 64, 256)
    np.testing.assert_array_equal(out.float().cpu().numpy(), codec.round_to_bf16(x))


@pytest.mark.parametrize("yarn", [False, True])
def test_rope_table(yarn):
    need_gpu()
    rows = 1 << 20
    cos, sin = rope_tables(rows, yarn=yarn)
    om = rope.frequencies(160000.0, rope.V4_YARN if yarn else None)
    pos = np.array([0, 1, 2, 127, 128, 4096, 65535, 65536, 262143, 524287, rows - 1])
    ang = rope.angles(pos, om)
    c = cos.cpu().numpy()[pos]
    s = sin.cpu().numpy()[pos]
    # one rounding of the float64 values to float32 (allow one ulp for libm differences)
    assert np.max(np.abs(c - np.cos(ang))) <= 1.2e-7
    assert np.max(np.abs(s - np.sin(ang))) <= 1.2e-7
