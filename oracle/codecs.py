"""Storage codecs: bfloat16 and OCP FP8 E4M3 ("e4m3fn").

Test infrastructure (see the package docstring); not imported by the library.

The design page "Distributed Layerwise Offload" (section "Feature
compatibility", row "Per-tensor online FP8 linears", and section "Request and
loading constraints") keeps fp8 linear weights together with one scale per
tensor, finalised before the blocks are offloaded.  The codecs below are the
plain definitions of the two formats:

* bfloat16: the top 16 bits of an IEEE binary32; encoding rounds to nearest,
  ties to the even 16-bit pattern.
* E4M3 (OCP 8-bit floating point, "FN" variant): sign, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); no
  infinities; S.1111.111 is NaN; largest finite magnitude 1.75 * 2^8 = 448.

Encoders here pick the nearest representable value by comparing distances
in float64 against an explicit table, which is a different route from the
library's bit manipulation.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# ---------------------------------------------------------------- bfloat16

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bf16 patterns, round to nearest, ties to even.

    For each finite value the two neighbouring bf16 values (toward zero and
    away from zero) are formed and the nearer one is kept; on a tie the one
    whose last mantissa bit is 0 wins.  NaN maps to the quiet NaN 0x7FC0
    with the sign kept; infinities stay infinities."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    toward = (u & np.uint32(0xFFFF0000))                 # truncation: toward zero
    away = toward + np.uint32(0x10000)                    # next pattern away from zero
    xv = x.astype(np.float64)
    t_val = toward.view(np.float32).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        a_val = away.view(np.float32).astype(np.float64)
        # past the largest finite value the next pattern is infinity; as a grid
        # point it stands at 2^128, so magnitudes from the midpoint up round to
        # infinity (IEEE 754 round to nearest on overflow)
        a_val = np.where(np.isinf(a_val) & np.isfinite(xv), np.copysign(2.0 ** 128, xv), a_val)
        d_t = np.abs(xv - t_val)
        d_a = np.abs(a_val - xv)
    t_hi = (toward >> np.uint32(16)).astype(np.uint16)
    a_hi = (away >> np.uint32(16)).astype(np.uint16)
    pick_away = (d_a < d_t) | ((d_a == d_t) & ((t_hi & np.uint16(1)) == 1))
    out = np.where(pick_away, a_hi, t_hi).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)).astype(np.uint16) & np.uint16(0x8000)) | np.uint16(0x7FC0)
    inf = np.isinf(x)
    if inf.any():
        out[inf] = (u[inf] >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> float64 value of its bf16 rounding."""
    return bf16_decode(bf16_encode(x))


def bf16_round_grid(x: np.ndarray) -> np.ndarray:
    """float32 -> float64 value of its bf16 rounding, from the format's grid
    instead of its bit patterns: bf16 keeps 8 significant bits, so inside the
    binade [2^(E-1), 2^E) (``frexp``'s exponent E) its values are the
    multiples of 2^(E-8), and below the smallest normal 2^-126 the multiples
    of 2^-133.  The value is the nearest multiple, ties to the even multiple
    (``rint``), which is the even mantissa pattern; a magnitude that rounds to
    2^128 or more overflows to infinity.  All of it is exact in float64.  The
    same values as ``bf16_round`` (pinned bit for bit), several times faster
    on the hundreds of millions of weights of a large block."""
    xv = np.asarray(x, dtype=np.float32).astype(np.float64)
    _, e = np.frexp(xv)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    with np.errstate(invalid="ignore", over="ignore"):
        v = np.rint(xv / q) * q
        v = np.where(np.abs(v) >= 2.0 ** 128, np.copysign(np.inf, xv), v)
    return v


# ---------------------------------------------------------------- fp8 e4m3

def _e4m3_table() -> np.ndarray:
    """Value of every code 0..255 (float64; NaN for the two NaN codes)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()
_POS = E4M3_VALUES[:127]          # codes 0..126: 0 .. 448, increasing


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float -> e4m3 codes: nearest value, ties to the even code, magnitudes
    above 448 saturate to 448; the sign bit follows the input's sign (a
    negative value that rounds to zero gives 0x80).  NaN gives 0x7F."""
    xv = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(xv), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")           # _POS[hi-1] < a <= _POS[hi]
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(xv).astype(np.uint8) << 7
    out = (mag | sign).astype(np.uint8)
    nan = np.isnan(xv)
    if nan.any():
        out[nan] = 0x7F
    return out


def e4m3_round_grid(x: np.ndarray) -> np.ndarray:
    """float -> float64 value of its e4m3 rounding (as e4m3_decode(e4m3_encode(x))),
    from the format's grid: magnitudes are first saturated to 448; inside the
    binade [2^(E-1), 2^E) the values are the multiples of 2^(E-4) (3 mantissa
    bits), below the smallest normal 2^-6 the multiples of 2^-9 (the
    subnormals m/8 * 2^-6); the nearest multiple is taken, ties to the even
    one (the even code).  The sign is kept; NaN stays NaN."""
    xv = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(xv), E4M3_MAX)
    _, e = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(e - 4, -9))
    with np.errstate(invalid="ignore"):
        return np.copysign(np.rint(a / q) * q, xv)


def quantize_tensor_e4m3(w: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Per-tensor scaling: s = amax(|w|) / 448 in float32 (1.0 for an all-zero
    tensor); codes = e4m3(w / s) with the division done in float32."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0.0)
    s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    q = (w / s).astype(np.float32)
    return e4m3_encode(q), s


def quantize_rows_e4m3(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Dynamic per-row activation scaling, taken entirely in float32:
    amax_r = max|x_r|, s_r = amax_r / 448, codes = e4m3(x_r * (448 / amax_r));
    an all-zero row gets s_r = 1 and zero codes."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1).astype(np.float32)
    nz = amax > 0
    s = np.where(nz, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0)).astype(np.float32)
    inv = np.where(nz, (np.float32(E4M3_MAX) / np.where(nz, amax, np.float32(1.0))).astype(np.float32),
                   np.float32(0.0)).astype(np.float32)
    q = (x * inv[..., None]).astype(np.float32)
    return e4m3_encode(q), s
