"""KV-cache row codecs (oracle).  Test infrastructure only.

Pages:
* V4-Flash model record (phantomic12.github.io), engine-constraint notes: the
  FP8 decode layout is 512 e4m3 values plus 16 e8m0 scales, one per 32 values
  (528 B per row); the FP4 layout is 288 B per row.
* V4.1-Flash diagram (flozi.net), "four compression axes": main KV in MXFP4,
  E2M1 values with one E4M3 scale per 16 channels; the sliding-window KV stays
  FP8.
* "DeepSeek-V4 deep dive", section 4.2 notes: FP8 rounding uses power-of-two
  (UE8M0) scales.

Readings where the pages are silent (all listed in the design notes):
* e4m3 is OCP E4M3FN: bias 7, largest finite 448, no infinities, NaN is
  S.1111.111.  Rounding is round-to-nearest-even, subnormals kept, finite
  overflow saturates to +-448.  NaN and +-Inf inputs encode as NaN
  (sign kept) so that they propagate.
* FP8-MX32 group = 32 consecutive dims.  Scale 2**e with e the smallest
  integer such that amax <= 448 * 2**e (amax over the finite values of the
  group), clamped to [-127, 127]; amax == 0 gives e = -127.  Scale byte is
  e + 127.  Row = D code bytes followed by D/32 scale bytes.
* MXFP4-E4M3/16 group = 16 consecutive dims.  Scale = e4m3(RNE(fp32(amax) /
  fp32(6))) computed in IEEE float32; a group holding NaN/Inf gets the NaN
  scale byte (0x7F) and zero codes.  Code = RNE onto the E2M1 grid
  {0, .5, 1, 1.5, 2, 3, 4, 6} of fp32(x) / fp32(scale), ties to the even
  code, saturating at 6, sign bit = sign of x; a zero scale gives all-zero
  codes.  Element 2j sits in the low nibble of byte j.  Row = D/2 code bytes
  followed by D/16 scale bytes.
* bf16 is the top half of an IEEE float32, rounded to nearest even.

FP4 indexer keys ("DeepSeek-V4 deep dive", section 5.2 implementation notes:
index keys and queries in MXFP4 after the Hadamard rotation; the OCP MX
format, E2M1 elements with one E8M0 scale per 32):
* MXFP4-MX32 group = 32 consecutive dims.  Shared exponent X =
  floor(log2(amax)) - 2 (2 is E2M1's largest exponent), clamped to
  [-127, 127]; amax == 0 gives X = -127.  Code = RNE onto the E2M1 grid of
  x / 2**X, ties to the even code, saturating at 6.  A group holding NaN/Inf
  gets the E8M0 NaN byte 0xFF and zero codes.  Element 2j sits in the low
  nibble of byte j.  Row = D/2 code bytes followed by D/32 scale bytes
  (X + 127): 68 B per 128-d key.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


# ----------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x):
    """RNE float32 -> bf16 bit patterns (uint16).  NaN stays NaN."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f64(b):
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_to_bf16(x):
    """Value of RNE-to-bf16 of float32(x), as float64."""
    return bf16_bits_to_f64(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


# ----------------------------------------------------------------------------
# e4m3 (OCP E4M3FN)
# ----------------------------------------------------------------------------

def e4m3_decode(code):
    """uint8 codes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    E = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(E == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (E - 7.0))
    val = np.where((E == 15) & (m == 7), np.nan, val)
    return s * val


def e4m3_encode(y):
    """RNE encode of float64 values into e4m3 codes (uint8), saturating.

    For |y| >= 2**-6 the exponent E = floor(log2 |y|) is read exactly with
    frexp and the significand |y| / 2**E in [1, 2) is rounded to 3 fraction
    bits; below that the value is rounded to a multiple of 2**-9.  Both
    scalings are by powers of two, hence exact.
    """
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros(y.shape, dtype=np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.abs(y)
    finite = np.isfinite(y)
    a0 = np.where(finite, a, 0.0)
    # subnormal / small branch
    small = a0 < 2.0 ** -6
    k = np.rint(np.where(small, a0, 0.0) * 512.0)  # 0..8 (8 == smallest normal, code 0x08)
    # normal branch
    f, ex = np.frexp(np.where(small, 1.0, a0))  # a = f * 2**ex, f in [0.5, 1)
    E = ex.astype(np.int64) - 1
    q = np.rint(f * 16.0).astype(np.int64)  # significand * 8, in [8, 16]
    carry = q == 16
    E = np.where(carry, E + 1, E)
    q = np.where(carry, 8, q)
    code_n = ((E + 7) << 3) | (q - 8)
    sat = (E > 8) | ((E == 8) & (q > 14))
    code_n = np.where(sat, 0x7E, code_n)
    code = np.where(small, k.astype(np.int64), code_n)
    code = np.where(finite, code, E4M3_NAN)
    out[...] = (code.astype(np.uint8) | sign)
    return out


# ----------------------------------------------------------------------------
# FP8-MX32 rows (528 B per 512-d row, 132 B per 128-d row)
# ----------------------------------------------------------------------------

def mx32_exponent(amax):
    """Smallest integer e with amax <= 448 * 2**e, clamped to [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    f, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    E = ex.astype(np.int64) - 1
    mant = f * 2.0  # in [1, 2)
    e = E - 8 + (mant > 1.75).astype(np.int64)
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127)


def fp8_mx32_row_bytes(dim):
    return dim + dim // 32


def quantize_fp8_mx32(x):
    """x: [..., D] float (f32-representable) -> uint8 [..., D + D/32]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % 32 == 0
    g = x.reshape(x.shape[:-1] + (D // 32, 32))
    fin = np.isfinite(g)
    amax = np.max(np.where(fin, np.abs(g), 0.0), axis=-1)
    e = mx32_exponent(amax)
    y = g * np.exp2(-e.astype(np.float64))[..., None]
    codes = e4m3_encode(y).reshape(x.shape[:-1] + (D,))
    scales = (e + 127).astype(np.uint8)
    return np.concatenate([codes, scales], axis=-1)


def dequantize_fp8_mx32(row, dim):
    row = np.asarray(row, dtype=np.uint8)
    codes = row[..., :dim]
    sc = row[..., dim:dim + dim // 32].astype(np.int64) - 127
    v = e4m3_decode(codes).reshape(row.shape[:-1] + (dim // 32, 32))
    v = v * np.exp2(sc.astype(np.float64))[..., None]
    return v.reshape(row.shape[:-1] + (dim,))


# ----------------------------------------------------------------------------
# MXFP4 with E4M3 scale per 16 (288 B per 512-d row)
# ----------------------------------------------------------------------------

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def e2m1_encode(v):
    """RNE onto the E2M1 grid, ties to the even code, saturating at 6."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    c = np.searchsorted(_E2M1_MID, a, side="left")  # midpoints strictly below a
    at_mid = np.zeros(a.shape, dtype=bool)
    inb = c < len(_E2M1_MID)
    at_mid[inb] = a[inb] == _E2M1_MID[c[inb]]
    c = np.where(at_mid & (c % 2 == 1), c + 1, c)
    sign = np.signbit(v).astype(np.int64) << 3
    return (c | sign).astype(np.uint8)


def e2m1_decode(code):
    c = np.asarray(code, dtype=np.int64)
    return np.where(c & 8, -1.0, 1.0) * E2M1_GRID[c & 7]


def fp4_row_bytes(dim):
    return dim // 2 + dim // 16


def quantize_fp4_e4m3_16(x):
    """x: [..., D] float32-representable -> uint8 [..., D/2 + D/16]."""
    x32 = np.asarray(x, dtype=np.float32)
    D = x32.shape[-1]
    assert D % 32 == 0
    g = x32.reshape(x32.shape[:-1] + (D // 16, 16))
    fin = np.isfinite(g)
    allfin = np.all(fin, axis=-1)
    amax = np.max(np.where(fin, np.abs(g), np.float32(0)), axis=-1).astype(np.float32)
    s32 = (amax / np.float32(6.0)).astype(np.float32)  # IEEE float32 division
    scode = e4m3_encode(s32.astype(np.float64))
    scode = np.where(allfin, scode, E4M3_NAN).astype(np.uint8)
    sval = e4m3_decode(scode).astype(np.float32)  # exact
    safe = np.where((sval > 0) & allfin, sval, np.float32(1.0)).astype(np.float32)
    v = (g / safe[..., None]).astype(np.float32)  # IEEE float32 division
    codes = e2m1_encode(v.astype(np.float64))
    codes = np.where(((sval > 0) & allfin)[..., None], codes, 0).astype(np.uint8)
    codes = codes.reshape(x32.shape[:-1] + (D,))
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return np.concatenate([packed, scode], axis=-1)


def dequantize_fp4_e4m3_16(row, dim):
    row = np.asarray(row, dtype=np.uint8)
    packed = row[..., :dim // 2].astype(np.int64)
    codes = np.empty(row.shape[:-1] + (dim,), dtype=np.int64)
    codes[..., 0::2] = packed & 0xF
    codes[..., 1::2] = packed >> 4
    sc = e4m3_decode(row[..., dim // 2:dim // 2 + dim // 16])
    v = e2m1_decode(codes).reshape(row.shape[:-1] + (dim // 16, 16)) * sc[..., None]
    return v.reshape(row.shape[:-1] + (dim,))


# ----------------------------------------------------------------------------
# MXFP4 with E8M0 scale per 32 (OCP MX FP4): 68 B per 128-d index key
# ----------------------------------------------------------------------------

def mx4_exponent(amax):
    """floor(log2(amax)) - 2, clamped to [-127, 127]; amax == 0 gives -127."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = ex.astype(np.int64) - 1 - 2
    X = np.where(amax > 0, X, -127)
    return np.clip(X, -127, 127)


def fp4_mx32_row_bytes(dim):
    return dim // 2 + dim // 32


def quantize_fp4_mx32(x):
    """x: [..., D] float32-representable -> uint8 [..., D/2 + D/32]."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    D = x.shape[-1]
    assert D % 32 == 0
    g = x.reshape(x.shape[:-1] + (D // 32, 32))
    fin = np.isfinite(g)
    allfin = np.all(fin, axis=-1)
    amax = np.max(np.where(fin, np.abs(g), 0.0), axis=-1)
    X = mx4_exponent(amax)
    y = np.where(fin, g, 0.0) * np.exp2(-X.astype(np.float64))[..., None]
    codes = np.where(allfin[..., None], e2m1_encode(y), 0).astype(np.uint8)
    codes = codes.reshape(x.shape[:-1] + (D,))
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    scales = np.where(allfin, X + 127, 0xFF).astype(np.uint8)
    return np.concatenate([packed, scales], axis=-1)


def dequantize_fp4_mx32(row, dim):
    row = np.asarray(row, dtype=np.uint8)
    packed = row[..., :dim // 2].astype(np.int64)
    codes = np.empty(row.shape[:-1] + (dim,), dtype=np.int64)
    codes[..., 0::2] = packed & 0xF
    codes[..., 1::2] = packed >> 4
    sb = row[..., dim // 2:dim // 2 + dim // 32].astype(np.int64)
    sc = np.where(sb == 0xFF, np.nan, np.exp2((sb - 127).astype(np.float64)))
    v = e2m1_decode(codes).reshape(row.shape[:-1] + (dim // 32, 32)) * sc[..., None]
    return v.reshape(row.shape[:-1] + (dim,))


# ----------------------------------------------------------------------------
# generic helpers
# ----------------------------------------------------------------------------

# ----------------------------------------------------------------------------
# V4 mixed rows: 448 NoPE dims in FP8, the 64 RoPE dims in bf16 ("DeepSeek-V4
# deep dive" sections 3.1 and 3.3 notes: 448 + 64 x 2 = 576 bytes, scale bytes
# not counted; the NoPE dims are rounded to FP8 in blocks of 64)
# ----------------------------------------------------------------------------

MIX_NOPE = 448
MIX_GROUP = 64
MIX_ROW_BYTES = 592  # 448 codes + 128 bf16 bytes + 7 E8M0 scales, padded to 16 B


def quantize_mix576(x):
    """x: [..., 512] float (f32-representable) -> uint8 [..., 592]: E4M3 codes
    of dims 0..447 with one E8M0 scale per 64 (the MX rule: the smallest e with
    amax <= 448 * 2**e), the bf16 bits (RNE) of dims 448..511, the 7 scale
    bytes e + 127, then 9 zero bytes."""
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == 512
    lead = x.shape[:-1]
    g = x[..., :MIX_NOPE].reshape(lead + (MIX_NOPE // MIX_GROUP, MIX_GROUP))
    amax = np.max(np.where(np.isfinite(g), np.abs(g), 0.0), axis=-1)
    e = mx32_exponent(amax)
    codes = e4m3_encode(g * np.exp2(-e.astype(np.float64))[..., None]).reshape(lead + (MIX_NOPE,))
    rope_bits = f32_to_bf16_bits(x[..., MIX_NOPE:].astype(np.float32))
    rope_bytes = np.ascontiguousarray(rope_bits.astype("<u2")).view(np.uint8).reshape(lead + (128,))
    scales = (e + 127).astype(np.uint8)
    pad = np.zeros(lead + (MIX_ROW_BYTES - 576 - 7,), np.uint8)
    return np.concatenate([codes.astype(np.uint8), rope_bytes, scales, pad], axis=-1)


def dequantize_mix576(row):
    row = np.asarray(row, dtype=np.uint8)
    lead = row.shape[:-1]
    sc = row[..., 576:583].astype(np.int64) - 127
    v = e4m3_decode(row[..., :MIX_NOPE]).reshape(lead + (7, MIX_GROUP))
    nope = (v * np.exp2(sc.astype(np.float64))[..., None]).reshape(lead + (MIX_NOPE,))
    bits = np.ascontiguousarray(row[..., MIX_NOPE:576]).view("<u2").reshape(lead + (64,))
    return np.concatenate([nope, bf16_bits_to_f64(bits)], axis=-1)


FORMATS = ("f32", "bf16", "fp8_mx32", "fp4_e4m3_16", "fp4_mx32", "mix576")


def row_bytes(fmt, dim):
    if fmt == "mix576":
        assert dim == 512
        return MIX_ROW_BYTES
    return {"f32": 4 * dim, "bf16": 2 * dim, "fp8_mx32": fp8_mx32_row_bytes(dim),
            "fp4_e4m3_16": fp4_row_bytes(dim), "fp4_mx32": fp4_mx32_row_bytes(dim)}[fmt]


def store(x, fmt):
    """Storage rounding: returns (stored representation, decoded float64)."""
    x = np.asarray(x, dtype=np.float64)
    if fmt == "f32":
        s = x.astype(np.float32)
        return s, s.astype(np.float64)
    if fmt == "bf16":
        b = f32_to_bf16_bits(x.astype(np.float32))
        return b, bf16_bits_to_f64(b)
    if fmt == "fp8_mx32":
        r = quantize_fp8_mx32(x.astype(np.float32).astype(np.float64))
        return r, dequantize_fp8_mx32(r, x.shape[-1])
    if fmt == "fp4_e4m3_16":
        r = quantize_fp4_e4m3_16(x.astype(np.float32))
        return r, dequantize_fp4_e4m3_16(r, x.shape[-1])
    if fmt == "fp4_mx32":
        r = quantize_fp4_mx32(x.astype(np.float32))
        return r, dequantize_fp4_mx32(r, x.shape[-1])
    if fmt == "mix576":
        r = quantize_mix576(x.astype(np.float32).astype(np.float64))
        return r, dequantize_mix576(r)
    raise ValueError(fmt)


def load(stored, fmt, dim):
    """Decode a stored representation back to float64 values."""
    if fmt == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(stored)
    if fmt == "fp8_mx32":
        return dequantize_fp8_mx32(stored, dim)
    if fmt == "fp4_e4m3_16":
        return dequantize_fp4_e4m3_16(stored, dim)
    if fmt == "fp4_mx32":
        return dequantize_fp4_mx32(stored, dim)
    if fmt == "mix576":
        return dequantize_mix576(stored)
    raise ValueError(fmt)
