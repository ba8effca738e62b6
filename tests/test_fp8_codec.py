"""Pins for the oracle's E4M3 codec and scale rule (O3), CPU only.

Pinned to an independent library (torch.float8_e4m3fn), to values read off
the OCP 8-bit floating point specification's E4M3 definition, and to hand-
worked rounding cases.
"""
import numpy as np
import pytest
import torch

from oracle import fp8 as O3


def test_decode_table_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O3.decode_table()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    # exactly two NaN codes (0x7F, 0xFF) in the fn variant
    assert sorted(np.flatnonzero(nan).tolist()) == [0x7F, 0xFF]


def test_spec_spot_values():
    # from the E4M3 row of the OCP FP8 specification: bias 7, max 448,
    # smallest subnormal 2^-9, smallest normal 2^-6.
    t = O3.decode_table()
    assert t[0x00] == 0.0
    assert t[0x01] == 2.0 ** -9
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0x08] == 2.0 ** -6
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0
    assert t[0xFE] == -448.0
    assert t[0x80] == 0.0 and np.signbit(t[0x80])


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        rng.uniform(-448, 448, 20000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-2).astype(np.float32),
    ])
    # every representable value and every midpoint between neighbours
    pos = O3.decode_table()[:127]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, pos.astype(np.float32), mids, -mids])
    ours = O3.encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_ties_round_to_even_code():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38.
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A): even code 0x3A.
    # 2^-10 lies halfway between 0 and 2^-9 (0x01): even code 0x00.
    # 3*2^-10 lies halfway between 2^-9 (0x01) and 2^-8 (0x02): 0x02.
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, -1.0625], np.float32)
    assert O3.encode(x).tolist() == [0x38, 0x3A, 0x00, 0x02, 0xB8]


def test_saturation_and_specials():
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e9, -1e9, np.inf, -np.inf, -0.0, 0.0, np.nan],
                 np.float32)
    assert O3.encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE,
                                     0x80, 0x00, 0x7F]


def test_scale_rule():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((33, 3, 16)).astype(np.float32)
    x[:, 2, :] = 0.0                                # all-zero head -> scale 1
    codes, s = O3.quantize_segment(x)
    assert s.dtype == np.float32
    amax = np.abs(x).max(axis=(0, 2))
    assert s[2] == 1.0 and (codes[:, 2, :] & 0x7F == 0).all()
    for h in range(2):
        assert s[h] == np.float32(amax[h]) / np.float32(448.0)
        # the element of largest magnitude lands on +-448 (code 0x7E / 0xFE)
        i = np.unravel_index(np.abs(x[:, h, :]).argmax(), x[:, h, :].shape)
        assert codes[i[0], h, i[1]] & 0x7F == 0x7E
    # round trip error is bounded by half an ulp of e4m3 (relative 2^-4) times
    # the scale, plus the subnormal spacing near zero
    y = O3.dequantize_segment(codes, s)
    err = np.abs(y - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s[None, :, None])
    assert (err <= bound + 1e-12).all()


def test_roundtrip_is_idempotent_on_the_grid():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 2, 8)).astype(np.float32)
    y = O3.roundtrip_segment(x)
    codes, s = O3.quantize_segment(x)
    # re-quantising the dequantised values with the same scale gives the same
    # codes
    again = O3.encode((y / s[None, :, None]).astype(np.float32))
    np.testing.assert_array_equal(again, codes)


def test_quantize_segment_matches_torch_fp32_pipeline():
    # the whole rule computed with torch's float32 ops and its e4m3 cast:
    # s = amax/448 (float32), codes = e4m3(x / s) with float32 division.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((257, 4, 32)) * rng.uniform(0.01, 30, (1, 4, 1))).astype(np.float32)
    codes, s = O3.quantize_segment(x)
    tx = torch.from_numpy(x)
    ts = tx.abs().amax(dim=(0, 2)) / torch.tensor(448.0, dtype=torch.float32)
    np.testing.assert_array_equal(s, ts.numpy())
    ref = (tx / ts[None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)


def test_division_is_float32_at_a_crafted_midpoint():
    # Pick x so that fl32(x / s) is exactly the midpoint 1.0625 between codes
    # 0x38 (1.0) and 0x39 (1.125) while the exact quotient lies above it.  The
    # float32 rule then ties to the even code 0x38; a float64 division would
    # round up to 0x39.
    amax = np.float32(300.0)
    s = amax / np.float32(448.0)
    target = np.float32(1.0625)
    x = np.float32(target * s)
    found = None
    for _ in range(64):
        q32 = np.float32(x / s)
        exact = float(x) / float(s)
        if q32 == target and exact > float(target):
            found = x
            break
        x = np.nextafter(x, np.float32(np.inf))
    assert found is not None
    seg = np.zeros((2, 1, 4), np.float32)
    seg[0, 0, 0] = amax
    seg[1, 0, 1] = found
    codes, sc = O3.quantize_segment(seg)
    assert sc[0] == s
    assert codes[1, 0, 1] == 0x38
