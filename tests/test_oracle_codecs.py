"""Pins for the oracle's FP8 E4M3 / ue8m0 / bf16 codecs (exhaustive, brute force, closed form)."""
import numpy as np


def test_fp8_decode_known_codes(orc):
    # OCP e4m3fn: bias 7, 3 mantissa bits, max 448, S.1111.111 = NaN
    d = orc.fp8_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0x80, 0xFE, 0x7F, 0xFF]))
    assert d[0] == 0.0 and d[1] == 2.0 ** -9 and d[2] == 7 * 2.0 ** -9
    assert d[3] == 2.0 ** -6 and d[4] == 1.0 and d[5] == 1.5 and d[6] == 448.0
    assert d[7] == 0.0 and np.signbit(d[7]) and d[8] == -448.0
    assert np.isnan(d[9]) and np.isnan(d[10])


def test_fp8_all_codes_roundtrip(orc):
    codes = np.arange(256, dtype=np.uint8)
    fin = (codes & 0x7F) != 0x7F
    vals = orc.fp8_decode(codes)
    assert np.array_equal(orc.fp8_encode(vals[fin]), codes[fin])
    # the 126 positive finite non-zero values are strictly increasing
    pos = vals[1:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_fp8_encode_matches_bruteforce_on_midpoints_and_random(orc):
    vals = orc.fp8_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    eps = np.abs(mids) * 1e-12 + 1e-300
    rng = np.random.default_rng(0)
    rnd = rng.standard_normal(200_000) * 2.0 ** rng.integers(-14, 10, 200_000)
    x = np.concatenate([mids, mids + eps, mids - eps, -mids, rnd, [0.0, -0.0, 447.9, 448.0, 460.0, 1e6, -1e6]])
    assert np.array_equal(orc.fp8_encode(x), orc.fp8_encode(x, brute=True))


def test_fp8_ties_to_even(orc):
    vals = orc.fp8_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    c = orc.fp8_encode(mids).astype(int)
    assert np.all(c % 2 == 0)


def test_fp8_saturates(orc):
    assert list(orc.fp8_encode(np.array([448.0, 1000.0, -1e30, np.inf, -np.inf]))) == [0x7E, 0x7E, 0xFE, 0x7E, 0xFE]


def test_ue8m0_boundaries(orc):
    k = np.arange(-20, 20)
    exact = 448.0 * 2.0 ** k
    assert np.array_equal(orc.ue8m0(exact), 2.0 ** k)
    assert np.array_equal(orc.ue8m0(exact * (1 + 2.0 ** -23)), 2.0 ** (k + 1))
    assert np.array_equal(orc.ue8m0(exact * (1 - 2.0 ** -23)), 2.0 ** k)
    assert orc.ue8m0(np.array([0.0]))[0] == 1.0


def test_ue8m0_is_smallest_power(orc):
    rng = np.random.default_rng(1)
    a = rng.random(10000) * 2.0 ** rng.integers(-30, 30, 10000) + 1e-30
    s = orc.ue8m0(a)
    assert np.all(np.log2(s) == np.round(np.log2(s)))
    assert np.all(a <= 448.0 * s) and np.all(a > 224.0 * s)


def test_bf16_rne_against_float32_bit_rounding(orc):
    rng = np.random.default_rng(2)
    f = (rng.standard_normal(100000) * 2.0 ** rng.integers(-40, 40, 100000)).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    ref = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(orc.bf16_from_double(f.astype(np.float64)), ref)


def test_bf16_no_double_rounding(orc):
    # 1 + 2^-8 + 2^-30: just above the bf16 midpoint 1 + 2^-8 -> must round up to 1 + 2^-7
    # (a float32 step first would land on the midpoint and round to even = 1.0)
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    h = orc.bf16_from_double(np.array([x]))[0]
    assert orc.bf16_to_double(np.array([h]))[0] == 1.0 + 2.0 ** -7
    assert orc.bf16_to_double(orc.bf16_from_double(np.array([1.0 + 2.0 ** -8])))[0] == 1.0


def test_quant_block_is_scaled_rne(orc):
    import dsa_inputs as gi
    x = gi.normal_bf16(7, 1, 0, 128 * 64).reshape(64, 128)
    codes, scale = orc.quant_fp8(x)
    xd = orc.bf16_to_double(x)
    amax = np.abs(xd).max(1)
    assert np.array_equal(scale.astype(np.float64), orc.ue8m0(amax))
    assert np.array_equal(codes, orc.fp8_encode(xd / scale[:, None].astype(np.float64), brute=True))
    # the block max lands in the top binade: no code above 448, none of the block uses less than half
    assert np.all(np.abs(orc.fp8_decode(codes)).max(1) > 224 * 0.9)
