"""Pins for O5 (rotary encoding of Q and K), CPU only.  Each test pins the
oracle to something other than itself: complex multiplication (numpy's
complex128), closed forms, the relative-position property of RoPE, and for
the stored bf16 values torch's float32 CPU arithmetic and a rounding written
from the definition on exact rationals (with a case where rounding once,
straight to bf16, would give a different value)."""
import math
from fractions import Fraction

import numpy as np
import torch

from oracle import attention as O1
from oracle import rope as O5


def test_rotation_is_complex_multiplication():
    # pair (x, y) as x + iy times cos + i sin (catches a sign or a swapped
    # pair member)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 8))
    ang = rng.uniform(-math.pi, math.pi, (5, 4))
    tab = np.stack([np.cos(ang), np.sin(ang)], axis=-1)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)[:, None, :]
    got = O5.rotate(x, tab)
    np.testing.assert_allclose(got[..., 0::2], z.real, atol=1e-14)
    np.testing.assert_allclose(got[..., 1::2], z.imag, atol=1e-14)


def test_special_angles():
    x = np.arange(1, 9, dtype=np.float64).reshape(1, 1, 8)
    ident = np.tile([1.0, 0.0], (1, 4, 1))
    np.testing.assert_array_equal(O5.rotate(x, ident), x)
    quarter = np.tile([0.0, 1.0], (1, 4, 1))        # (x, y) -> (-y, x)
    np.testing.assert_array_equal(O5.rotate(x, quarter)[0, 0], [-2, 1, -4, 3, -6, 5, -8, 7])


def test_rotation_keeps_pair_norms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 2, 16))
    tab = O5.table_1d(np.arange(7) * 3.5, 16)
    y = O5.rotate(x, tab)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)


def test_attention_depends_on_relative_positions_only():
    # shifting every query and key position by the same amount leaves the
    # attention output unchanged (the defining property of RoPE)
    rng = np.random.default_rng(2)
    n, S, H, d = 6, 10, 2, 16
    q = rng.standard_normal((n, H, d))
    k = rng.standard_normal((S, H, d))
    v = rng.standard_normal((S, H, d))
    pq = np.arange(n) + 40.0
    pk = np.arange(S) * 2.0
    out = []
    for shift in (0.0, 17.0, -123.5):
        qr = O5.rotate(q, O5.table_1d(pq + shift, d))
        kr = O5.rotate(k, O5.table_1d(pk + shift, d))
        out.append(O1.softmax_attention(qr, kr, v, 0.25)[0])
    np.testing.assert_allclose(out[1], out[0], atol=1e-12)
    np.testing.assert_allclose(out[2], out[0], atol=1e-12)
    # and the positions do matter (a wrong table would pass the test above
    # if it ignored them)
    qr = O5.rotate(q, O5.table_1d(pq, d))
    kr = O5.rotate(k, O5.table_1d(pk * 3.0, d))
    assert np.abs(O1.softmax_attention(qr, kr, v, 0.25)[0] - out[0]).max() > 1e-3


def test_stored_values_are_float32_ops_rounded_to_bf16():
    # against torch's float32 CPU arithmetic (separately rounded products,
    # then the sum/difference), then torch's bf16 cast
    g = torch.Generator().manual_seed(3)
    x = torch.randn(9, 4, 64, generator=g).to(torch.bfloat16)
    ang = torch.rand(9, 32, generator=g, dtype=torch.float64) * 6.3 - 3.15
    tab = torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).to(torch.float32)
    xf = x.to(torch.float32)
    c = tab[:, None, :, 0]
    s = tab[:, None, :, 1]
    ref = torch.empty_like(xf)
    ref[..., 0::2] = xf[..., 0::2] * c - xf[..., 1::2] * s
    ref[..., 1::2] = xf[..., 0::2] * s + xf[..., 1::2] * c
    got = O5.rotate_stored(x, tab.numpy())
    assert torch.equal(got.view(torch.int16), ref.to(torch.bfloat16).view(torch.int16))
    # and within one bf16 rounding of the exact rotation
    exact = O5.rotate(x, tab.numpy().astype(np.float64))
    assert np.abs(got.to(torch.float64).numpy() - exact).max() <= \
        2.0 ** -8 * np.abs(exact).max()


# Round to nearest, ties to even, into a binary format with p significand
# bits and smallest normal exponent emin (subnormals below it), written from
# the definition on exact rationals: independent of numpy's and torch's
# float32 and bf16 arithmetic.
def _rne(q: Fraction, p: int, emin: int) -> Fraction:
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, emin) - (p - 1))
    m = a / quantum
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return (1 if q > 0 else -1) * n * quantum


def _f32(q):
    return _rne(q, 24, -126)


def _bf16(q):
    return _rne(q, 8, -126)


def _stored_exact(xe, xo, c, s):
    """the pair's stored values: float32 products, float32 difference / sum,
    then bf16, every rounding on exact rationals"""
    xe, xo, c, s = (Fraction(float(v)) for v in (xe, xo, c, s))
    a, b = _f32(xe * c), _f32(xo * s)
    even = _bf16(_f32(a - b))
    a, b = _f32(xe * s), _f32(xo * c)
    odd = _bf16(_f32(a + b))
    return even, odd


def test_stored_values_match_exact_rational_rounding():
    # random pairs and angles
    g = torch.Generator().manual_seed(11)
    x = torch.randn(6, 2, 32, generator=g).to(torch.bfloat16)
    ang = torch.rand(6, 16, generator=g, dtype=torch.float64) * 6.3 - 3.15
    tab = torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).to(torch.float32).numpy()
    got = O5.rotate_stored(x, tab).to(torch.float64).numpy()
    xf = x.to(torch.float32).numpy()
    for r in range(x.shape[0]):
        for h in range(x.shape[1]):
            for i in range(x.shape[2] // 2):
                even, odd = _stored_exact(xf[r, h, 2 * i], xf[r, h, 2 * i + 1],
                                          tab[r, i, 0], tab[r, i, 1])
                assert Fraction(float(got[r, h, 2 * i])) == even
                assert Fraction(float(got[r, h, 2 * i + 1])) == odd


def test_stored_values_round_twice():
    # x = (1, 2^-10), (cos, sin) = (1 + 2^-8, -2^-20): the exact even
    # output is 1 + 2^-8 + 2^-30.  Rounded straight to bf16 it would be
    # 1 + 2^-7 (above the midpoint); through float32 it is first the
    # midpoint 1 + 2^-8, which bf16 rounds to even: 1.  The odd output is
    # sin + 2^-10 cos = -2^-20 + 2^-10 + 2^-18 (float32 exact), bf16 2^-10.
    x = torch.tensor([[[1.0, 2.0 ** -10]]], dtype=torch.bfloat16)
    tab = np.array([[[1.0 + 2.0 ** -8, -2.0 ** -20]]], dtype=np.float32)
    got = O5.rotate_stored(x, tab).to(torch.float64).numpy()[0, 0]
    assert got[0] == 1.0
    assert _bf16(Fraction(1) + Fraction(1, 2 ** 8) + Fraction(1, 2 ** 30)) == 1 + Fraction(1, 2 ** 7)
    assert (Fraction(float(got[0])), Fraction(float(got[1]))) == \
        _stored_exact(1.0, 2.0 ** -10, tab[0, 0, 0], tab[0, 0, 1])
    assert got[1] == 2.0 ** -10
