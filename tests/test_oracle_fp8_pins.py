"""Pins for the oracle's FP8 latent-cache functions (E4M3 codes, one
power-of-two scale per 1 x 128 tile).

Expected values come from the E4M3 definition worked by hand, from torch's own
float8_e4m3fn conversion (an implementation the oracle does not use), and from
the rounding error bound of a 3-bit mantissa.
"""
import numpy as np
import torch

from oracle import mla_oracle as om


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_value_table():
    """Facts of the format: 254 finite codes, 448 at 0x7E, 1.0 at 0x38, the
    smallest subnormal 2^-9 at 0x01, the smallest normal 2^-6 at 0x08, NaN at
    0x7F and 0xFF, sign-symmetric, increasing over 0x00..0x7E."""
    v = om.e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.isfinite(v).sum() == 254
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x7E] == 448.0 and v[0x38] == 1.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x07] == 7 * 2.0 ** -9 and v[0x39] == 1.125 and v[0x40] == 2.0
    assert np.all(np.diff(v[:0x7F]) > 0)
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])
    # torch's decoding of every code
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    fin = np.isfinite(v)
    assert np.array_equal(np.isnan(t), ~fin) and np.array_equal(t[fin], v[fin])


def test_e4m3_encode_round_trip_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    v = om.e4m3_value(codes)
    fin = np.isfinite(v)
    assert np.array_equal(om.e4m3_encode(v[fin]), codes[fin])
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(100000) * 2.0 ** rng.integers(-14, 8, 100000)).astype(np.float32)
    x = np.clip(x, -448, 448)
    assert np.array_equal(om.e4m3_encode(x), _torch_codes(x))


def test_e4m3_ties_to_even():
    """The midpoint of two neighbouring values takes the even code; a value
    just above (below) it takes the upper (lower) neighbour."""
    v = om.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2
    even = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    assert np.array_equal(om.e4m3_encode(mid), even.astype(np.uint8))
    assert np.array_equal(om.e4m3_encode(np.nextafter(mid, np.inf)), np.arange(1, 0x7F, dtype=np.uint8))
    assert np.array_equal(om.e4m3_encode(np.nextafter(mid, -np.inf)), np.arange(0x7E, dtype=np.uint8))
    assert om.e4m3_encode(np.array([-1e-9]))[0] == 0x80  # sign kept on a value rounding to zero


def test_fp8_tile_exponent():
    e = om.fp8_tile_exponent(np.array([448.0, 448.0 * (1 + 2.0 ** -40), 224.0, 224.0 * (1 + 2.0 ** -40), 10.0,
                                       0.0, 1.0, 2.0 ** -30]))
    # 10 / 2^-5 = 320 <= 448 < 640 = 10 / 2^-6; 1 / 2^-8 = 256; 2^-30 / 2^-38 = 256
    assert list(e) == [0, 1, -1, 0, -5, 0, -8, -38]
    rng = np.random.default_rng(6)
    a = np.abs(rng.standard_normal(10000)) * 2.0 ** rng.integers(-20, 20, 10000)
    r = a / 2.0 ** om.fp8_tile_exponent(a)
    assert np.all(r <= 448) and np.all(r > 224)


def test_quantize_worked_example():
    """One tile by hand: max |x| = 10 gives e = -5 (scale 1/32).
    1.0 -> 32 = 2^5: exponent field 12, code 0x60.
    10  -> 320 = 1.25 * 2^8: field 15, mantissa 2, code 0x7A.
    0.3 -> 9.6, spacing 1 in [8, 16): 10 = 1.25 * 2^3, code 0x52, back to 0.3125.
    1e-4 -> 0.0032 = 1.6384 * 2^-9 (subnormal): 2 * 2^-9, code 0x02, back to 2^-13."""
    x = np.zeros(128)
    x[:5] = [1.0, 10.0, 0.3, -0.3, 1e-4]
    codes, e, deq = om.quantize_latent_fp8(x[None])
    assert e.tolist() == [[-5]]
    assert codes[0, :5].tolist() == [0x60, 0x7A, 0x52, 0xD2, 0x02]
    assert np.allclose(deq[0, :5], [1.0, 10.0, 0.3125, -0.3125, 2.0 ** -13], rtol=0, atol=0)
    assert np.all(codes[0, 5:] == 0)


def test_quantize_error_bound_and_tiles():
    """Half a spacing at most: 2^(k-4) * scale in binade [2^k, 2^(k+1)) of
    x / scale (k >= -6), 2^-10 * scale below; every tile has its own scale."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((40, 512)) * np.repeat(2.0 ** rng.integers(-6, 6, (40, 4)), 128, axis=1)
    codes, e, deq = om.quantize_latent_fp8(x)
    x32 = x.astype(np.float32).astype(np.float64)
    s = np.repeat(2.0 ** e, 128, axis=1)
    a = np.abs(x32) / s
    k = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    assert np.all(np.abs(deq - x32) <= 2.0 ** (k - 4) * s)
    assert np.array_equal(deq, om.e4m3_value(codes) * s)
    for t in range(4):
        assert np.array_equal(e[:, t], om.fp8_tile_exponent(np.max(np.abs(x32[:, 128 * t:128 * t + 128]), axis=1)))
    assert np.array_equal(codes, _torch_codes(x32 / s))


def test_cache_row_fp8_matches_bf16_row_within_fp8_error():
    rng = np.random.default_rng(8)
    c_raw = rng.standard_normal((6, 512))
    k_raw = rng.standard_normal((6, 64))
    g = 1 + 0.3 * rng.standard_normal(512)
    pos = np.arange(100, 106)
    exact = om.cache_row(c_raw, k_raw, g, pos, 1e-6, 10000.0)
    codes, e, k_r, row = om.cache_row_fp8(c_raw, k_raw, g, pos, 1e-6, 10000.0)
    assert np.array_equal(row[:, 512:], exact[:, 512:]) and np.array_equal(k_r, exact[:, 512:])
    rel = np.abs(row[:, :512] - exact[:, :512]) / np.abs(exact[:, :512])
    big = np.abs(exact[:, :512]) / np.repeat(2.0 ** e, 128, axis=1) >= 2.0 ** -6
    assert rel[big].max() <= 2.0 ** -4 + 1e-7
