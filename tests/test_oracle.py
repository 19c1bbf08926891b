"""Pins for the CPU oracle: each check compares it with something other than
itself -- closed forms, the bf16 format definition, exact integer products
from NumPy, SciPy's logistic function, a hand-worked example, and a
pure-Python brute force -- so that a dropped term, a wrong sign, a wrong
index, a transposed operand or a swapped gate/up pairing fails a test."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import brute
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 decode
# Values fixed by the bfloat16 format (sign, 8-bit exponent bias 127, 7-bit
# mantissa): the oracle must widen these patterns exactly.
BF16_PATTERNS = [
    (0x0000, 0.0), (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0x3F00, 0.5),
    (0x4049, 3.140625), (0xC0A0, -5.0), (0x0080, 2.0 ** -126), (0x0001, 2.0 ** -133),
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127), (0x3F81, 1.0 + 2.0 ** -7),
]


@pytest.mark.parametrize("bits,value", BF16_PATTERNS)
def test_bf16_decode_format_values(bits, value):
    assert oracle.bf16_to_double(bits) == value


def test_bf16_decode_specials():
    assert oracle.bf16_to_double(0x7F80) == math.inf
    assert oracle.bf16_to_double(0xFF80) == -math.inf
    assert math.isnan(oracle.bf16_to_double(0x7FC0))
    z = oracle.bf16_to_double(0x8000)
    assert z == 0.0 and math.copysign(1.0, z) < 0


# ---------------------------------------------------------------- SiLU
def test_silu_zero_and_sigmoid_half():
    assert oracle.silu(0.0) == 0.0
    assert oracle.sigmoid(0.0) == 0.5


@pytest.mark.parametrize("a", [3.0, 1.0 / 3.0, 7.0, 99.0, 1e-3, 2.5e4])
def test_silu_closed_form_at_log(a):
    # sigmoid(ln a) = a / (1 + a) exactly, so silu(ln a) = ln(a) * a / (1 + a)
    z = math.log(a)
    assert oracle.silu(z) == pytest.approx(z * a / (1.0 + a), rel=1e-15, abs=1e-300)


def test_silu_matches_scipy_logistic_and_tanh_form():
    zs = np.linspace(-40.0, 40.0, 4001)
    ref = zs * scipy.special.expit(zs)
    got = np.array([oracle.silu(z) for z in zs])
    np.testing.assert_allclose(got, ref, rtol=2e-15, atol=1e-300)
    # silu(z) = (z / 2) * (1 + tanh(z / 2)); 1 + tanh cancels for z << 0, so
    # this form is only compared where it stays well conditioned.
    keep = zs >= -8.0
    ref2 = 0.5 * zs[keep] * (1.0 + np.tanh(0.5 * zs[keep]))
    np.testing.assert_allclose(got[keep], ref2, rtol=1e-12, atol=1e-300)


def test_silu_odd_part_identity():
    # sigmoid(z) + sigmoid(-z) = 1  =>  silu(z) - silu(-z) = z
    for z in np.linspace(-20, 20, 801):
        assert oracle.silu(z) - oracle.silu(-z) == pytest.approx(z, abs=1e-13)


def test_silu_limits_do_not_overflow():
    assert oracle.silu(800.0) == 800.0          # sigmoid -> 1
    v = oracle.silu(-800.0)                      # sigmoid -> 0, no NaN
    assert v == 0.0 or (v < 0 and abs(v) < 1e-300)
    assert oracle.silu(50.0) == pytest.approx(50.0, rel=1e-15)
    assert oracle.silu(-50.0) == pytest.approx(-50.0 * math.exp(-50.0), rel=1e-12)
    # silu'(z) = s(z) (1 + z (1 - s(z))) vanishes where s(z) = 1 + 1/z, so the
    # minimum value is z* + 1 with z* the root of 1 + z (1 - expit(z)) = 0.
    import scipy.optimize
    zstar = scipy.optimize.brentq(lambda z: 1 + z * (1 - scipy.special.expit(z)), -3, -0.5,
                                  xtol=1e-15)
    assert oracle.silu(zstar) == pytest.approx(zstar + 1.0, abs=1e-14)
    zs = np.linspace(-3, 0, 30001)
    assert min(oracle.silu(z) for z in zs) >= zstar + 1.0 - 1e-15


# ---------------------------------------------------------------- products
def _decode(a):
    return a.astype(np.float64) if a.dtype == np.float32 else wl.bf16_bits_to_f32(a).astype(np.float64)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 37, 29), (5, 64, 48), (2, 300, 700)])
def test_integer_products_exact(dtype, shape):
    M, d, dff = shape
    inp = wl.integer_inputs(7 + M + d, M, d, dff, dtype)
    h, g, u = oracle.swiglu(inp["x"], inp["wg"], inp["wu"], want_gu=True)
    xi = _decode(inp["x"]).astype(np.int64)
    gi = xi @ _decode(inp["wg"]).astype(np.int64)
    ui = xi @ _decode(inp["wu"]).astype(np.int64)
    assert np.array_equal(g, gi.astype(np.float64))
    assert np.array_equal(u, ui.astype(np.float64))
    ref = gi * scipy.special.expit(gi.astype(np.float64)) * ui
    np.testing.assert_allclose(h, ref, rtol=4e-15, atol=0)


def test_gate_up_orientation():
    # Swapping the roles of Wgate and Wup must change the result; with
    # Wgate == Wup the result is silu(g) * g.
    inp = wl.integer_inputs(3, 4, 16, 24, wl.F32)
    h1 = oracle.swiglu(inp["x"], inp["wg"], inp["wu"])
    h2 = oracle.swiglu(inp["x"], inp["wu"], inp["wg"])
    assert not np.allclose(h1, h2)
    hs, g, _ = oracle.swiglu(inp["x"], inp["wg"], inp["wg"], want_gu=True)
    np.testing.assert_allclose(hs, g * g * scipy.special.expit(g), rtol=4e-15, atol=0)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_one_hot_rows_select_weight_rows(dtype):
    d, dff = 40, 33
    ks = [0, 17, 39, 5]
    x = wl.one_hot_rows(len(ks), d, ks, dtype)
    w = wl.random_inputs(11, 1, d, dff, dtype)
    h, g, u = oracle.swiglu(x, w["wg"], w["wu"], want_gu=True)
    wg, wu = _decode(w["wg"]), _decode(w["wu"])
    for m, k in enumerate(ks):
        assert np.array_equal(g[m], wg[k])
        assert np.array_equal(u[m], wu[k])
        np.testing.assert_allclose(h[m], wg[k] * scipy.special.expit(wg[k]) * wu[k],
                                   rtol=4e-15, atol=0)


def test_zero_input_gives_zero():
    w = wl.random_inputs(5, 3, 24, 40, wl.BF16, with_down=True)
    x = np.zeros_like(w["x"])
    h = oracle.swiglu(x, w["wg"], w["wu"])
    y = oracle.mlp(x, w["wg"], w["wu"], w["wd"])
    assert not h.any() and not y.any()
    # Wup = 0 also gives zero
    assert not oracle.swiglu(w["x"], w["wg"], np.zeros_like(w["wu"])).any()


def test_down_projection_one_hot_columns():
    M, d, dff = 3, 12, 20
    w = wl.random_inputs(21, M, d, dff, wl.F32)
    cols = [19, 0, 7, 7, 3, 11, 15, 2, 9, 1, 18, 4]     # Wd[:, j] = e_{cols[j]}
    wd = np.zeros((dff, d), dtype=np.float32)
    for j, n in enumerate(cols):
        wd[n, j] = 1.0
    y, h = oracle.mlp(w["x"], w["wg"], w["wu"], wd, want_h=True)
    for j, n in enumerate(cols):
        assert np.array_equal(y[:, j], h[:, n])


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_down_projection_integer(dtype):
    M, d, dff = 4, 24, 56
    inp = wl.integer_inputs(9, M, d, dff, dtype, with_down=True, lo=-2, hi=2)
    y = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"])
    xi = _decode(inp["x"]).astype(np.int64)
    g = (xi @ _decode(inp["wg"]).astype(np.int64)).astype(np.float64)
    u = (xi @ _decode(inp["wu"]).astype(np.int64)).astype(np.float64)
    ref = (g * scipy.special.expit(g) * u) @ _decode(inp["wd"])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "tiny_integer_example.json")) as f:
        ex = json.load(f)
    x, wg, wu, wd = (np.array(ex[k], dtype=np.float32) for k in ("x", "wg", "wu", "wd"))
    y, h = oracle.mlp(x, wg, wu, wd, want_h=True)
    _, g, u = oracle.swiglu(x, wg, wu, want_gu=True)
    assert np.array_equal(g, np.array(ex["g_by_hand"], dtype=np.float64))
    assert np.array_equal(u, np.array(ex["u_by_hand"], dtype=np.float64))
    gh = np.array(ex["g_by_hand"], dtype=np.float64)
    np.testing.assert_allclose(h, gh * scipy.special.expit(gh) * np.array(ex["u_by_hand"]),
                               rtol=4e-15)
    np.testing.assert_allclose(y[:, 0], h[:, 0], rtol=0)
    np.testing.assert_allclose(y[:, 1], 2 * h[:, 1], rtol=0)
    np.testing.assert_allclose(y[:, 2], -h[:, 0] + h[:, 1], rtol=1e-15)


# ---------------------------------------------------------------- oracle vs brute force
@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("shape", [(1, 3, 2), (2, 5, 7), (3, 8, 4), (4, 6, 9)])
def test_c_oracle_matches_pure_python(dtype, shape):
    M, d, dff = shape
    inp = wl.random_inputs(100 + d, M, d, dff, dtype, with_down=True)
    xs, gs, us, ds = (_decode(inp[k]).tolist() for k in ("x", "wg", "wu", "wd"))
    h_ref = np.array(brute.swiglu(xs, gs, us))
    y_ref = np.array(brute.mlp(xs, gs, us, ds))
    y, h = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"], want_h=True)
    np.testing.assert_allclose(h, h_ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(y, y_ref, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- harness properties
def test_row_subset_and_thread_count_are_bitwise_stable():
    inp = wl.random_inputs(77, 9, 96, 1100, wl.BF16, with_down=True)
    full = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"], nthreads=1)
    par = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"], nthreads=4)
    sub = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"], rows=[8, 2, 5], nthreads=3)
    assert np.array_equal(full, par)
    assert np.array_equal(sub, full[[8, 2, 5]])


def test_bad_arguments_rejected():
    inp = wl.random_inputs(1, 2, 8, 8, wl.F32)
    with pytest.raises(ValueError):
        oracle.swiglu(inp["x"], inp["wg"], inp["wu"], rows=[2])
    with pytest.raises(TypeError):
        oracle.swiglu(inp["x"].astype(np.float64), inp["wg"], inp["wu"])
