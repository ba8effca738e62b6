"""O3: OCP FP8 E4M3 codec and the per-(head, segment) scale rule.

Test infrastructure only (see the package docstring).

The pages only say that the deployment runs in FP8 (discuss.pytorch.kr,
"JoyAI-Video-Edit 소개", real-time deployment section; ta-paperlens section 5);
they do not say which tensors or which format.  The reading used here, for a
K/V cache stored in 8 bits:

* format: OCP 8-bit floating point, E4M3 ("fn" variant: no infinities, one NaN
  mantissa pattern per sign, largest finite magnitude 448, exponent bias 7,
  subnormals down to 2^-9);
* scale: one float32 per (head, stored segment): s = amax / 448 computed in
  float32, where amax is the largest magnitude of that head's values in the
  segment; s = 1 when amax = 0;
* code: e4m3(x / s), with x / s a correctly rounded float32 division, rounded
  to the nearest representable E4M3 value, ties to the even code, saturating
  at +-448; the sign bit of x is kept (so -0.0 and tiny negatives give 0x80);
* dequantised value: value(code) * s, exact in float64.

Encoding searches the sorted table of representable magnitudes; it performs
no bit tricks, so it can be checked against the format definition by eye.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes, from the E4M3 definition.

    code = s eeee mmm: e = 0 -> (-1)^s * (m/8) * 2^-6 (subnormal);
    e > 0 -> (-1)^s * (1 + m/8) * 2^(e-7); e = 15 and m = 7 -> NaN.
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = (code >> 7) & 1
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            v = np.nan
        elif e == 0:
            v = (m / 8.0) * 2.0 ** -6
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals[code] = -v if s else v
    return vals


_TABLE = decode_table()
_POS = _TABLE[:127]          # codes 0x00..0x7E: 0 .. 448, strictly increasing


def encode(x) -> np.ndarray:
    """Round float32 values to E4M3 codes (nearest, ties to even, saturating)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    sign = np.signbit(x).astype(np.uint8) << 7
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    mag = np.where(_POS[hi] == a, hi, mag).astype(np.uint8)
    codes = (mag | sign).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F) | sign, codes).astype(np.uint8)


def decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def segment_scales(x) -> np.ndarray:
    """float32 scale per head for one stored segment x [rows, H, d]."""
    x = np.asarray(x, dtype=np.float32)
    H = x.shape[1]
    amax = np.abs(x).transpose(1, 0, 2).reshape(H, -1).max(axis=1) if x.shape[0] else \
        np.zeros(H, np.float32)
    amax = amax.astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0))
    return s.astype(np.float32)


def quantize_segment(x):
    """Codes [rows, H, d] uint8 and scales [H] float32 for one segment."""
    x = np.asarray(x, dtype=np.float32)
    s = segment_scales(x)
    y = (x / s[None, :, None]).astype(np.float32)     # float32 division
    return encode(y), s


def dequantize_segment(codes, scales) -> np.ndarray:
    """Exact float64 values code * scale, [rows, H, d]."""
    return decode(codes) * np.asarray(scales, np.float64)[None, :, None]


def roundtrip_segment(x) -> np.ndarray:
    """dq(q(x)): the float64 values an fp8 cache holds for x [rows, H, d]."""
    codes, s = quantize_segment(x)
    return dequantize_segment(codes, s)
