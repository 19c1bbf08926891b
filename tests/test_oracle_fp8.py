"""Pins for the oracle's FP8 (OCP E4M3, no infinities) weight format and its
per-column quantiser, each against something other than the oracle itself:
the format's constants (largest value 448, smallest subnormal 2^-9,
smallest normal 2^-6, NaN at S.1111.111), a brute-force nearest search over
all finite values, grids on which quantisation must be exact, fp32 scale
arithmetic redone in NumPy, and the error bound that round-to-nearest with
three mantissa bits guarantees."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

# (code, value) fixed by the format: sign, exponent bias 7, 3 mantissa bits
E4M3_VALUES = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x02, 2.0 ** -8), (0x07, 7 * 2.0 ** -9),
    (0x08, 2.0 ** -6), (0x0F, 1.875 * 2.0 ** -6), (0x30, 0.5), (0x38, 1.0),
    (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x4B, 5.5), (0x70, 128.0),
    (0x77, 240.0), (0x78, 256.0), (0x7D, 416.0), (0x7E, 448.0),
    (0x81, -(2.0 ** -9)), (0xB8, -1.0), (0xFE, -448.0),
]


@pytest.mark.parametrize("code,value", E4M3_VALUES)
def test_e4m3_decode_format_values(code, value):
    assert oracle.e4m3_to_double(code) == value


def test_e4m3_decode_specials_order_and_symmetry():
    assert math.isnan(oracle.e4m3_to_double(0x7F))
    assert math.isnan(oracle.e4m3_to_double(0xFF))
    z = oracle.e4m3_to_double(0x80)
    assert z == 0.0 and math.copysign(1.0, z) == -1.0
    pos = [oracle.e4m3_to_double(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:])), "codes 0x00..0x7E increase"
    for c in range(0x7F):
        assert oracle.e4m3_to_double(c | 0x80) == -pos[c]
    # 0x08 starts the normal range where the subnormals end (7 * 2^-9 + 2^-9)
    assert pos[8] - pos[7] == 2.0 ** -9


def test_e4m3_encode_round_trips_every_finite_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_from_float(oracle.e4m3_to_double(c)) == c, hex(c)


_GRID = []   # the non-negative finite values, filled on first use


def _brute_nearest(v: float) -> int:
    """Nearest finite E4M3 code by exhaustive search; a tie goes to the even
    code; the sign is carried separately (so -0.0 and tiny negatives give
    0x80)."""
    if not _GRID:
        _GRID.extend(Fraction(oracle.e4m3_to_double(c)) for c in range(0x7F))
    a = Fraction(abs(v))                    # exact: every value here is dyadic
    dist = [abs(g - a) for g in _GRID]
    low = min(dist)
    best = [c for c in range(0x7F) if dist[c] == low]
    code = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
    return code | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_e4m3_encode_matches_brute_force_nearest():
    rng = np.random.default_rng(8)
    mags = np.exp2(rng.uniform(-13, 10, 3000)).astype(np.float32)
    vals = (mags * rng.choice([-1, 1], mags.size)).astype(np.float32)
    # every midpoint between neighbouring values, and points just off them
    grid = [oracle.e4m3_to_double(c) for c in range(0x7F)]
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]
    extra = []
    for m in mids:
        f = np.float32(m)
        extra += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1e9))]
    extra += [np.float32(v) for v in (0.0, -0.0, 448.0, 448.5, 464.0, 479.9, 1e6, -1e30, 2.0 ** -12)]
    for v in list(vals) + extra:
        assert oracle.e4m3_from_float(v) == _brute_nearest(float(v)), float(v)


@pytest.mark.parametrize("v,code", [
    (1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
    (7.5 * 2.0 ** -9, 0x08), (432.0, 0x7E), (424.0, 0x7D), (460.0, 0x7E), (-1e9, 0xFE),
])
def test_e4m3_encode_ties_to_even_and_saturates(v, code):
    assert oracle.e4m3_from_float(v) == code


def test_quantize_is_exact_on_scaled_e4m3_grids():
    # w = s * e4m3(c) with s a power of two and one +-448 code per column:
    # bf16 holds these exactly, the scale comes out as s, and every code is
    # recovered.
    rng = np.random.default_rng(3)
    K, N = 40, 24
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    codes = rng.choice(finite, size=(K, N)).astype(np.uint8)
    codes[rng.integers(0, K, N), np.arange(N)] = rng.choice([0x7E, 0xFE], N)
    s = np.exp2(rng.integers(-12, 4, N)).astype(np.float32)
    dec = np.array([[oracle.e4m3_to_double(c) for c in row] for row in codes])
    w = wl.f32_to_bf16_bits((dec * s).astype(np.float32))
    assert np.array_equal(wl.bf16_bits_to_f32(w).astype(np.float64), dec * s)
    q, sc = oracle.quantize_e4m3(w)
    assert np.array_equal(sc, s)
    # -0.0 and +0.0 codes may both stand for zero; everything else must match
    zero = np.isin(codes, (0x00, 0x80))
    assert np.array_equal(np.where(zero, 0, q), np.where(zero, 0, codes))


def test_quantize_scale_arithmetic_and_error_bound():
    rng = np.random.default_rng(5)
    K, N = 300, 40
    wf = (rng.standard_normal((K, N)) * np.exp2(rng.integers(-6, 6, N))).astype(np.float32)
    wf[:, 7] = 0.0                        # an all-zero column
    wf[:5, 9] = [1e-3, -2e-3, 0.0, 5e-4, 3.0]
    w = wl.f32_to_bf16_bits(wf)
    wv = wl.bf16_bits_to_f32(w)
    q, s = oracle.quantize_e4m3(w)
    amax = np.abs(wv).max(axis=0).astype(np.float32)
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))
    assert s[7] == 0 and not q[:, 7].any()
    deq = oracle.dequantize_e4m3(q, s)
    # nearest-even with 3 mantissa bits: |error| <= 2^-4 |w| in the normal
    # range, <= 2^-10 * scale among subnormals; plus the fp32 division
    bound = 2.0 ** -4 * np.abs(wv) + 2.0 ** -10 * s + 2.0 ** -22 * np.abs(wv)
    assert np.all(np.abs(deq - wv) <= bound)
    # the largest magnitude of each column lands on +-448 exactly
    big = np.abs(wv).argmax(axis=0)
    for n in range(N):
        if s[n] > 0:
            assert q[big[n], n] in (0x7E, 0xFE)
            assert abs(deq[big[n], n]) == 448.0 * float(s[n])


def test_dequantize_is_scale_times_code_value():
    codes = np.array([[0x38, 0x7E], [0xB8, 0x01]], dtype=np.uint8)
    scales = np.array([0.5, 3.0], dtype=np.float32)
    assert np.array_equal(oracle.dequantize_e4m3(codes, scales),
                          np.array([[0.5, 1344.0], [-0.5, 3.0 * 2.0 ** -9]]))


def test_fp64_inputs_give_the_bf16_results_bitwise():
    # the fp64 input path reads the same values as the (pinned) bf16 path
    inp = wl.random_inputs(12, 3, 40, 24, wl.BF16, with_down=True)
    f = {k: oracle.bf16_array_to_double(v) for k, v in inp.items()}
    assert np.array_equal(oracle.swiglu(f["x"], f["wg"], f["wu"]),
                          oracle.swiglu(inp["x"], inp["wg"], inp["wu"]))
    assert np.array_equal(oracle.mlp(f["x"], f["wg"], f["wu"], f["wd"]),
                          oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"]))


def test_fp8_weight_mlp_on_a_hand_checked_case():
    # x = [1, 2]; Wg = [[1], [0.5]] (codes 0x38, 0x30, scale 1);
    # Wu = [[2], [-1]] (codes 0x40, 0xB8, scale 1): g = 2, u = 0
    # -> h = 0; and with Wu = [[2], [1]]: u = 4, h = silu(2) * 4
    x = wl.f32_to_bf16_bits(np.array([[1.0, 2.0]], dtype=np.float32))
    qg = np.array([[0x38], [0x30]], dtype=np.uint8)
    qu = np.array([[0x40], [0xB8]], dtype=np.uint8)
    one = np.ones(1, dtype=np.float32)
    assert oracle.swiglu_fp8w(x, qg, one, qu, one)[0, 0] == 0.0
    qu2 = np.array([[0x40], [0x38]], dtype=np.uint8)
    h = oracle.swiglu_fp8w(x, qg, one, qu2, one)[0, 0]
    assert abs(h - 2.0 / (1.0 + math.exp(-2.0)) * 4.0) < 1e-15
