"""Partial rotary position embedding (oracle, float64).

Test infrastructure only (see the package docstring).

Pages: "DeepSeek-V4 deep dive", section 3.3 (partial RoPE and the inverse
rotation on the output) and section 9.1 (YaRN settings table and the
correction-range formula in its implementation notes).

* Only the last 64 of the head dimensions carry position.  They are viewed as
  32 complex numbers made of adjacent pairs (dim 2k, dim 2k+1 of that slice),
  and pair k is multiplied by exp(i * p * omega_k).  The inverse rotation uses
  the conjugate, i.e. the angle -p * omega_k (section 3.3).
* Reading: omega_k = theta ** (-2k / 64), the usual RoPE frequency ladder.
  It is pinned by the wavelength table of section 9.1 (pairs 0, 15, 25, 31
  have wavelengths of about 6, 1,700, 73,000 and 691,000 tokens at base
  160,000).
* YaRN (section 9.1): factor 16 over 65,536 original positions, beta_fast 32,
  beta_slow 1.  The correction range is
  (floor(c(beta_fast)), ceil(c(beta_slow))) with
  c(beta) = 64 * ln(L0 / (2 pi beta)) / (2 ln theta), which the page
  evaluates to (15, 25).  Pairs below the range keep their frequency, pairs
  above it are divided by the factor, and a linear ramp blends in between:
  omega' = omega / factor * (1 - smooth) + omega * smooth,
  smooth = 1 - clamp((k - lo) / (hi - lo), 0, 1).
* No attention-temperature (mscale) factor (section 9.1 notes).
"""

import math

import numpy as np

ROPE_DIMS = 64
NPAIRS = ROPE_DIMS // 2


def yarn_correction_range(theta, orig_len, beta_fast=32.0, beta_slow=1.0, rope_dims=ROPE_DIMS):
    """(lo, hi) pair indices of the YaRN ramp (section 9.1 notes)."""

    def c(beta):
        return rope_dims * math.log(orig_len / (2.0 * math.pi * beta)) / (2.0 * math.log(theta))

    lo = math.floor(c(beta_fast))
    hi = math.ceil(c(beta_slow))
    lo = max(lo, 0)
    hi = min(hi, rope_dims // 2 - 1)
    return lo, hi


def frequencies(theta, yarn=None):
    """Return omega[32] (float64).

    yarn: None for plain RoPE, else a dict with keys factor, orig_len,
    beta_fast, beta_slow (section 9.1 table: 16, 65536, 32, 1).
    """
    k = np.arange(NPAIRS, dtype=np.float64)
    omega = theta ** (-2.0 * k / ROPE_DIMS)
    if yarn is not None:
        lo, hi = yarn_correction_range(theta, yarn["orig_len"], yarn.get("beta_fast", 32.0),
                                       yarn.get("beta_slow", 1.0))
        if hi == lo:
            hi = lo + 0.001
        ramp = np.clip((k - lo) / (hi - lo), 0.0, 1.0)
        smooth = 1.0 - ramp
        omega = omega / yarn["factor"] * (1.0 - smooth) + omega * smooth
    return omega


V4_YARN = {"factor": 16.0, "orig_len": 65536, "beta_fast": 32.0, "beta_slow": 1.0}


def angles(positions, omega):
    """angle[p, k] = p * omega_k in float64."""
    p = np.asarray(positions, dtype=np.float64)
    return p[..., None] * omega


def rotate(x, positions, omega, inverse=False):
    """Rotate the last 64 dims of x (float64 copy) at the given positions.

    x: [..., D] with D >= 64; positions broadcast against x[..., 0].
    Pair k is (x[D-64+2k], x[D-64+2k+1]) -> (a cos - b sin, a sin + b cos);
    the inverse uses -angle.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    D = x.shape[-1]
    ang = angles(positions, omega)
    if inverse:
        ang = -ang
    c = np.cos(ang)
    s = np.sin(ang)
    a = x[..., D - ROPE_DIMS + 0::2].copy()
    b = x[..., D - ROPE_DIMS + 1::2].copy()
    x[..., D - ROPE_DIMS + 0::2] = a * c - b * s
    x[..., D - ROPE_DIMS + 1::2] = a * s + b * c
    return x
