"""Pins for the oracle's MXFP4 weight format (OCP Microscaling v1.0: E2M1
elements, one E8M0 power-of-two scale per 32 consecutive K values), each
against something other than the oracle itself: the format's value table,
an exact brute-force nearest search, the shared-exponent rule checked as an
interval property, grids on which quantisation must be exact, and the error
bound of round-to-nearest with one mantissa bit."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_value_table():
    for c, v in enumerate(E2M1):
        assert oracle.e2m1_to_double(c) == v
        assert oracle.e2m1_to_double(c | 8) == -v
    assert math.copysign(1.0, oracle.e2m1_to_double(8)) == -1.0


def test_e2m1_round_trip_every_code():
    for c in range(16):
        assert oracle.e2m1_from_double(oracle.e2m1_to_double(c)) == c


def _brute(v: float) -> int:
    a = Fraction(abs(v))
    dist = [abs(Fraction(g) - a) for g in E2M1]
    low = min(dist)
    best = [c for c in range(8) if dist[c] == low]
    code = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
    return code | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_encode_matches_brute_force_nearest():
    rng = np.random.default_rng(2)
    vals = list(rng.uniform(-9, 9, 2000)) + list(np.exp2(rng.uniform(-6, 3, 500)))
    mids = [(a + b) / 2 for a, b in zip(E2M1, E2M1[1:])]
    for m in mids:
        vals += [m, -m, np.nextafter(m, 0.0), np.nextafter(m, 9.0)]
    vals += [0.0, -0.0, 6.0, 6.5, 7.0, 100.0, -1e30, 0.1]
    for v in vals:
        assert oracle.e2m1_from_double(float(v)) == _brute(float(v)), v


@pytest.mark.parametrize("v,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4),
                                    (3.5, 6), (5.0, 6), (5.5, 7), (6.5, 7), (-2.6, 13)])
def test_e2m1_ties_to_even_and_saturation(v, code):
    assert oracle.e2m1_from_double(v) == code


def test_non_finite_values_saturate_with_their_sign():
    # E2M1's value table has no infinity or NaN: the reading taken is that
    # they lie beyond 6 and saturate, keeping the sign bit
    assert oracle.e2m1_from_double(math.inf) == 7
    assert oracle.e2m1_from_double(-math.inf) == 15
    assert oracle.e2m1_from_double(math.nan) == 7
    assert oracle.e2m1_from_double(-math.nan) == 15
    # floor(log2(inf)) - 2 is infinite: the clamp's top
    assert oracle.mx_shared_exponent(math.inf) == 127


def test_nan_weight_does_not_set_the_block_exponent():
    w = wl.f32_to_bf16_bits(np.full((40, 2), 1.0, dtype=np.float32))
    w[5, 0] = 0x7FC0                        # NaN among ones
    w[:, 1] = 0
    w[33, 1] = 0xFF80                       # -inf alone in the ragged block
    q, sc = oracle.quantize_mxfp4(w)
    assert sc[0, 0] == 127 - 2 and q[5, 0] == 7 and q[4, 0] == 6   # 1.0 = 4 * 2^-2, code 6
    assert sc[1, 1] == 127 + 127 and q[33, 1] == 15 and sc[0, 1] == 127


def test_shared_exponent_puts_the_block_max_in_4_to_8():
    rng = np.random.default_rng(3)
    for amax in np.exp2(rng.uniform(-100, 100, 500)):
        s = oracle.mx_shared_exponent(amax)
        assert 4.0 <= amax / 2.0 ** s < 8.0
    assert oracle.mx_shared_exponent(1.0) == -2
    assert oracle.mx_shared_exponent(6.0) == 0
    assert oracle.mx_shared_exponent(0.0) == 0
    assert oracle.mx_shared_exponent(1e-40) == -126      # clamped: scales stay normal fp32


def test_quantize_is_exact_on_scaled_e2m1_grids():
    # each 32-row block holds 2^s * E2M1 values with one +-4 or +-6 element,
    # so the shared exponent is s and every code comes back
    rng = np.random.default_rng(4)
    K, N = 96, 10
    codes = rng.integers(0, 16, (K, N)).astype(np.uint8)
    s = rng.integers(-20, 5, (K // 32, N))
    for b in range(K // 32):
        codes[32 * b + rng.integers(0, 32), np.arange(N)] = rng.choice([6, 7, 14, 15], N)
    val = np.array([[oracle.e2m1_to_double(c) for c in row] for row in codes])
    w = val * np.exp2(np.repeat(s, 32, axis=0))
    wb = wl.f32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(wl.bf16_bits_to_f32(wb).astype(np.float64), w)
    q, sc = oracle.quantize_mxfp4(wb)
    assert np.array_equal(sc.astype(np.int64) - 127, s)
    zero = np.isin(codes, (0, 8))
    assert np.array_equal(np.where(zero, 0, q), np.where(zero, 0, codes))


def test_quantize_blocks_errors_and_zero_blocks():
    rng = np.random.default_rng(5)
    K, N = 70, 12                          # blocks of 32, 32 and a ragged 6
    wf = (rng.standard_normal((K, N)) * np.exp2(rng.integers(-8, 8, N))).astype(np.float32)
    wf[32:64, 3] = 0.0                      # an all-zero block
    w = wl.f32_to_bf16_bits(wf)
    wv = wl.bf16_bits_to_f32(w).astype(np.float64)
    q, sc = oracle.quantize_mxfp4(w)
    assert sc.shape == (3, N)
    assert sc[1, 3] == 127 and not (q[32:64, 3] & 7).any()
    deq = oracle.dequantize_mxfp4(q, sc)
    X = np.exp2(np.repeat(sc.astype(np.int64) - 127, 32, axis=0)[:K])
    inside = np.abs(wv) <= 6 * X
    # one mantissa bit, nearest: within a quarter of |w| plus a quarter of
    # the block scale (the subnormal step is X / 2); beyond 6 X, saturation
    assert np.all(np.abs(deq - wv)[inside] <= (0.25 * np.abs(wv) + 0.25 * X)[inside])
    assert np.all(np.abs(deq[~inside]) == 6 * X[~inside])
    for b in range(3):
        blk = np.abs(wv[32 * b:32 * b + 32])
        nz = blk.max(axis=0) > 0
        r = blk.max(axis=0)[nz] / X[32 * b][nz]
        assert np.all((4 <= r) & (r < 8))


def test_dequantize_is_power_of_two_scale_times_value():
    codes = np.array([[7], [9]] * 16 + [[2]], dtype=np.uint8)          # 33 rows: 2 blocks
    scales = np.array([[127 - 3], [127 + 2]], dtype=np.uint8)
    out = oracle.dequantize_mxfp4(codes, scales)
    assert out[0, 0] == 6.0 / 8 and out[1, 0] == -0.5 / 8 and out[32, 0] == 1.0 * 4
