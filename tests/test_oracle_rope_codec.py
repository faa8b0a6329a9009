"""Pins for the oracle's RoPE and codec (CPU only)."""

import math

import numpy as np
import pytest

from oracle import codec, rope


# ----------------------------------------------------------------------------- RoPE

def test_wavelengths_match_page_table(golden):
    g = golden["wavelengths"]
    om = rope.frequencies(160000.0)  # base frequencies, before YaRN
    lam = 2 * np.pi / om
    assert 5.5 <= lam[0] <= 6.5                       # "about 6"
    assert abs(lam[15] / g["pair15_about"] - 1) < 0.03  # "about 1,700"
    assert abs(lam[25] / g["pair25_about"] - 1) < 0.01  # "about 73,000"
    assert abs(lam[31] / g["pair31_about"] - 1) < 0.002  # "about 691,000"


def test_yarn_correction_range(golden):
    y = golden["yarn"]
    lo, hi = rope.yarn_correction_range(y["theta"], y["orig_len"], y["beta_fast"], y["beta_slow"])
    assert (lo, hi) == tuple(y["correction_range"])
    assert y["factor"] * y["orig_len"] == y["max_positions"]


def test_yarn_direction():
    base = rope.frequencies(160000.0)
    yr = rope.frequencies(160000.0, rope.V4_YARN)
    # pairs 0-15 unchanged, 25-31 divided by 16, in between strictly blended
    np.testing.assert_array_equal(yr[:16], base[:16])
    np.testing.assert_allclose(yr[25:], base[25:] / 16, rtol=1e-15)
    mid = yr[16:25] / base[16:25]
    assert np.all((mid < 1) & (mid > 1 / 16)) and np.all(np.diff(mid) < 0)


def test_relative_rotation_example(golden):
    g = golden["rope_relative"]
    om = np.zeros(32)
    om[0] = math.radians(g["theta_deg"])
    u = np.zeros(64)
    u[0] = 1.0
    for shift in (0, g["shift"]):
        stored = rope.rotate(u, g["key_pos"] + shift, om)
        back = rope.rotate(stored, g["query_pos"] + shift, om, inverse=True)
        ang = math.degrees(math.atan2(back[1], back[0]))
        assert abs(ang - g["net_deg"]) < 1e-9


def test_rotate_inverse_identity_and_nope_untouched():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 512))
    om = rope.frequencies(160000.0, rope.V4_YARN)
    y = rope.rotate(x, [5, 70000, 1048575], om)
    np.testing.assert_array_equal(y[:, :448], x[:, :448])
    z = rope.rotate(y, [5, 70000, 1048575], om, inverse=True)
    np.testing.assert_allclose(z, x, atol=1e-12)
    # pair layout: adjacent dims (448+2k, 449+2k) rotate together by p*omega_k
    p = 9
    e = np.zeros(512)
    e[448 + 2 * 7] = 1.0
    r = rope.rotate(e, p, om)
    assert abs(r[448 + 14] - math.cos(p * om[7])) < 1e-15
    assert abs(r[448 + 15] - math.sin(p * om[7])) < 1e-15


# ----------------------------------------------------------------------------- codec

def _all_finite_e4m3_values():
    codes = np.arange(256, dtype=np.uint8)
    vals = codec.e4m3_decode(codes)
    keep = np.isfinite(vals)
    return codes[keep], vals[keep]


def test_row_sizes(golden):
    assert codec.fp8_mx32_row_bytes(512) == golden["cache_bytes"]["fp8_row"] == 528
    assert codec.fp4_row_bytes(512) == golden["cache_bytes"]["fp4_row"] == 288
    assert codec.fp8_mx32_row_bytes(128) == 132
    x = np.random.default_rng(1).standard_normal((3, 512))
    assert codec.quantize_fp8_mx32(x).shape == (3, 528)
    assert codec.quantize_fp4_e4m3_16(x).shape == (3, 288)


def test_e4m3_decode_known_values():
    d = codec.e4m3_decode
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    codes, vals = _all_finite_e4m3_values()
    assert len(codes) == 254 and np.max(vals) == 448.0


def test_e4m3_roundtrip_all_codes():
    codes, vals = _all_finite_e4m3_values()
    back = codec.e4m3_encode(vals)
    np.testing.assert_array_equal(back, codes)


def test_e4m3_encode_is_nearest_even_bruteforce():
    codes, vals = _all_finite_e4m3_values()
    pos = codes < 0x80
    pc, pv = codes[pos], vals[pos]
    rng = np.random.default_rng(2)
    # random values, exact midpoints and saturating values
    ys = np.concatenate([rng.uniform(0, 460, 4000), rng.uniform(0, 2.0 ** -5, 2000),
                         (pv[:-1] + pv[1:]) / 2, [448.0, 460.0, 463.99, 1e6]])
    for y in ys:
        got = int(codec.e4m3_encode(np.array([y]))[0])
        dist = np.abs(pv - min(y, 448.0))
        best = np.flatnonzero(dist == dist.min())
        if len(best) == 1:
            want = int(pc[best[0]])
        else:  # tie: even mantissa (even code)
            want = int([pc[b] for b in best if pc[b] % 2 == 0][0])
        assert got == want, (y, got, want)
    assert int(codec.e4m3_encode(np.array([-1.0]))[0]) == 0xB8
    assert int(codec.e4m3_encode(np.array([np.nan]))[0]) == 0x7F
    assert int(codec.e4m3_encode(np.array([-np.inf]))[0]) == 0xFF


def test_e4m3_relative_error_bound():
    rng = np.random.default_rng(3)
    y = rng.uniform(2.0 ** -6, 448.0, 20000)
    back = codec.e4m3_decode(codec.e4m3_encode(y))
    assert np.max(np.abs(back - y) / y) <= 2.0 ** -4


def test_mx32_exponent_rule():
    e = codec.mx32_exponent
    assert e(448.0) == 0 and e(448.0001) == 1 and e(224.0) == -1 and e(1.0) == -8
    assert e(1.75) == -8 and e(1.76) == -7 and e(0.0) == -127 and e(1e-40) == -127
    # smallest e with amax <= 448 * 2**e, checked by search
    for a in np.random.default_rng(4).uniform(1e-6, 1e6, 500):
        k = int(e(a))
        assert a <= 448 * 2.0 ** k and not (a <= 448 * 2.0 ** (k - 1))


def test_fp8_mx32_row_layout_and_grid_roundtrip():
    rng = np.random.default_rng(5)
    codes, vals = _all_finite_e4m3_values()
    # a row whose groups hold grid values times 2**e with amax exactly 448 * 2**e
    x = rng.choice(vals[np.abs(vals) <= 448], size=(2, 512))
    x[:, ::32] = 448.0
    sc = rng.integers(-20, 20, size=(2, 16))
    x = (x.reshape(2, 16, 32) * np.exp2(sc)[..., None]).reshape(2, 512)
    r = codec.quantize_fp8_mx32(x)
    np.testing.assert_array_equal(r[:, 512:].astype(int) - 127, sc)
    np.testing.assert_array_equal(codec.dequantize_fp8_mx32(r, 512), x)


def test_e2m1_encode_bruteforce():
    grid = codec.E2M1_GRID
    rng = np.random.default_rng(6)
    ys = np.concatenate([rng.uniform(0, 7, 3000), (grid[:-1] + grid[1:]) / 2, [6.0, 6.5, 100.0]])
    for y in ys:
        got = int(codec.e2m1_encode(np.array([y]))[0])
        dist = np.abs(grid - min(y, 6.0))
        best = np.flatnonzero(dist == dist.min())
        want = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        assert got == want, (y, got, want)
    assert int(codec.e2m1_encode(np.array([-3.0]))[0]) == 0x8 | 5


def test_fp4_row_layout_and_grid_roundtrip():
    rng = np.random.default_rng(7)
    codes, vals = _all_finite_e4m3_values()
    # every group: E2M1 grid values with amax 6, times an e4m3 scale
    g = rng.choice(codec.E2M1_GRID, size=(3, 32, 16)) * rng.choice([-1, 1], size=(3, 32, 16))
    g[..., 0] = 6.0
    s = rng.choice(vals[(vals > 2 ** -6) & (vals < 64)], size=(3, 32))
    x = (g * s[..., None]).reshape(3, 512)
    r = codec.quantize_fp4_e4m3_16(x)
    np.testing.assert_array_equal(codec.e4m3_decode(r[:, 256:]), s)
    np.testing.assert_array_equal(codec.dequantize_fp4_e4m3_16(r, 512), x)
    # nibble order: element 2j in the low nibble of byte j
    one = np.zeros(512)
    one[0], one[1] = 6.0, -1.0
    rr = codec.quantize_fp4_e4m3_16(one)
    assert rr[0] == (7 | ((8 | 2) << 4))


def test_fp4_scale_rule_float32():
    x = np.zeros(512, np.float32)
    x[:16] = np.float32(1.0)
    r = codec.quantize_fp4_e4m3_16(x)
    # scale = RNE_e4m3(fp32(1)/6) = 0.171875 (0.1666.. lies between 0.15625 and 0.171875,
    # nearer the latter); 1/0.171875 = 5.818 -> code for 6
    assert codec.e4m3_decode(r[256]) == 0.171875
    assert (r[0] & 0xF) == 7
    # zero group -> zero scale and codes
    assert r[257] == 0 and r[8] == 0


def test_fp4_mx32_row_size_and_exponent_rule():
    # index keys of the FP4 indexer: 132 B (FP8) -> 68 B per 128-d key
    assert codec.fp4_mx32_row_bytes(128) == 68 and codec.row_bytes("fp4_mx32", 512) == 272
    # X = floor(log2 amax) - 2, brute force over exact powers of two
    for amax in [1.0, 1.5, 3.99, 4.0, 6.0, 7.9, 2.0 ** -100, 2.0 ** 100, 1e-45, 3e38]:
        want = max(-127, min(127, math.floor(math.log2(amax)) - 2))
        assert int(codec.mx4_exponent(np.array([amax]))[0]) == want, amax
    assert int(codec.mx4_exponent(np.array([0.0]))[0]) == -127


def test_fp4_mx32_codes_bruteforce_and_grid_roundtrip():
    rng = np.random.default_rng(8)
    grid = codec.E2M1_GRID
    # brute force: every element is the nearest grid value times 2**X, ties to
    # the even code, saturating at 6 * 2**X
    x = (rng.standard_normal((64, 128)) * rng.choice([1e-3, 1.0, 50.0], (64, 1))).astype(np.float32)
    r = codec.quantize_fp4_mx32(x)
    assert r.shape == (64, 68)
    v = codec.dequantize_fp4_mx32(r, 128)
    for i in range(64):
        for gi in range(4):
            grp = x[i, 32 * gi:32 * gi + 32].astype(np.float64)
            X = math.floor(math.log2(np.abs(grp).max())) - 2
            assert r[i, 64 + gi] == X + 127
            for j, y in enumerate(grp / 2.0 ** X):
                dist = np.abs(grid - min(abs(y), 6.0))
                best = np.flatnonzero(dist == dist.min())
                c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
                assert v[i, 32 * gi + j] == math.copysign(grid[c], y) * 2.0 ** X
    # grid values with an amax of 4 or 6 in the top binade survive exactly
    g = rng.choice(grid, size=(5, 4, 32)) * rng.choice([-1, 1], size=(5, 4, 32))
    g[..., 0] = rng.choice([4.0, 6.0], size=(5, 4))
    k = rng.integers(-20, 20, size=(5, 4))
    xg = (g * np.exp2(k)[..., None]).reshape(5, 128)
    np.testing.assert_array_equal(codec.dequantize_fp4_mx32(codec.quantize_fp4_mx32(xg), 128), xg)
    # saturation: amax 7 * 2**k has X = k and stores 6 * 2**k; zero group -> byte 0, codes 0
    z = np.zeros(128, np.float32)
    z[0] = 7.0 * 2 ** -3
    rz = codec.quantize_fp4_mx32(z)
    assert rz[64] == 127 - 3 and (rz[0] & 0xF) == 7 and rz[65] == 0 and not rz[16:32].any()
    assert codec.dequantize_fp4_mx32(rz, 128)[0] == 6.0 * 2 ** -3
    # non-finite group: NaN scale byte, zero codes, decodes to NaN
    z[40] = np.inf
    rn = codec.quantize_fp4_mx32(z)
    assert rn[65] == 0xFF and not rn[16:32].any()
    assert np.isnan(codec.dequantize_fp4_mx32(rn, 128)[32:64]).all()


def test_bf16_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    np.testing.assert_array_equal(codec.round_to_bf16(x),
                                  [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7])


def test_mix576_layout_and_rounding():
    """The V4 mixed row (deep dive sections 3.1 and 3.3 notes): 448 FP8 + 64
    bf16 = 576 bytes before scales, FP8 in blocks of 64.  The 64 RoPE dims are
    RNE bf16 bit patterns, exactly; every NoPE value decodes to the nearest
    E4M3 grid value of x / 2**e (brute force over all finite codes, ties to
    the even code) times 2**e, with e the smallest exponent that fits the
    block's amax under 448."""
    assert codec.MIX_NOPE * 1 + 64 * 2 == 576
    assert codec.row_bytes("mix576", 512) == 592 and 592 % 16 == 0
    rng = np.random.default_rng(21)
    x = rng.standard_normal((6, 512)) * np.exp2(rng.integers(-12, 12, (6, 1)))
    x[1, :64] = 0.0                       # an all-zero block
    x[2, 100] = 448.0 * 3.9               # a block whose amax sets a high scale
    x = x.astype(np.float32).astype(np.float64)
    row = codec.quantize_mix576(x)
    assert row.shape == (6, 592) and np.all(row[:, 583:] == 0)
    back = codec.dequantize_mix576(row)
    np.testing.assert_array_equal(back[:, 448:], codec.round_to_bf16(x[:, 448:]))
    bits = np.ascontiguousarray(row[:, 448:576]).view("<u2")
    np.testing.assert_array_equal(bits, codec.f32_to_bf16_bits(x[:, 448:].astype(np.float32)))
    grid = codec.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = np.isfinite(grid)
    codes = np.arange(256)[fin]
    vals = grid[fin]
    for r in range(6):
        for g in range(7):
            blk = x[r, 64 * g:64 * g + 64]
            amax = np.abs(blk).max()
            e = min(k for k in range(-127, 128) if amax <= 448.0 * 2.0 ** k)
            assert int(row[r, 576 + g]) - 127 == e, (r, g)
            for j in range(64):
                y = blk[j] * 2.0 ** -e
                d = np.abs(vals - y)
                best = np.flatnonzero(d == d.min())
                if len(best) > 1:  # tie: the even code
                    best = best[(codes[best] & 1) == 0]
                want = vals[best[0]] * 2.0 ** e
                assert back[r, 64 * g + j] == want or (want == 0 and back[r, 64 * g + j] == 0)
