"""Pins for the oracle's RMSNorm and the MLP half of a layer (RMSNorm
prologue, residual and bias epilogue), each against something other than
the oracle itself: rows whose norm has a closed form, exact power-of-two
scale invariance, a hand-worked example, a pure-Python brute force, and
weights that reduce the block to the residual or to the pinned MLP."""
import math

import numpy as np
import pytest

import oracle
import workloads as wl


def test_constant_rows_give_the_gain():
    # r_i = c: mean square c^2, so n_i = sign(c) * gamma_i (eps = 0)
    gamma = np.array([0.5, -2.0, 3.0, 1.25])
    for c in (1.0, -3.0, 7.5):
        n = oracle.rmsnorm(np.full((1, 4), c), gamma, 0.0)
        assert np.allclose(n[0], math.copysign(1.0, c) * gamma, rtol=1e-15, atol=0)


def test_one_hot_row_gives_sqrt_d():
    # r = a e_j: mean square a^2 / d, so n_j = sqrt(d) gamma_j sign(a), 0 elsewhere
    d = 64
    gamma = np.linspace(0.5, 2.0, d)
    r = np.zeros((1, d)); r[0, 9] = -5.0
    n = oracle.rmsnorm(r, gamma, 0.0)[0]
    assert abs(n[9] - (-math.sqrt(d) * gamma[9])) <= 1e-14 * math.sqrt(d) * gamma[9]
    assert not np.delete(n, 9).any()


def test_power_of_two_scaling_is_exact_without_eps():
    rng = np.random.default_rng(1)
    r = rng.standard_normal((3, 40))
    g = rng.standard_normal(40)
    assert np.array_equal(oracle.rmsnorm(r * 2.0 ** 7, g, 0.0), oracle.rmsnorm(r, g, 0.0))


def test_eps_closed_form_and_zero_rows():
    # d = 1: n = x / sqrt(x^2 + eps) * gamma
    for x, eps in ((0.3, 1e-2), (-2.0, 0.5), (1e-3, 1e-6)):
        n = oracle.rmsnorm(np.array([[x]]), np.array([2.0]), eps)[0, 0]
        assert abs(n - 2.0 * x / math.sqrt(x * x + eps)) <= 1e-15 * abs(n)
    assert not oracle.rmsnorm(np.zeros((2, 8)), np.ones(8), 1e-5).any()


def test_hand_worked_example():
    # r = [3, 4]: mean square 12.5, rms 5 / sqrt 2 -> n = [0.6, 0.8] * sqrt 2
    n = oracle.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 1.0]), 0.0)[0]
    assert np.allclose(n, [0.6 * math.sqrt(2), 0.8 * math.sqrt(2)], rtol=1e-15, atol=0)


def test_brute_force_and_storage_dtypes():
    rng = np.random.default_rng(4)
    r = rng.standard_normal((5, 24)).astype(np.float32)
    g = rng.standard_normal(24).astype(np.float32)
    eps = 1e-5
    want = [[float(r[m, i]) / math.sqrt(sum(float(v) ** 2 for v in r[m]) / 24 + eps) * float(g[i])
             for i in range(24)] for m in range(5)]
    assert np.allclose(oracle.rmsnorm(r, g, eps), want, rtol=1e-13, atol=0)
    # bf16 storage is widened exactly: same result as fp64 copies of the values
    rb, gb = wl.f32_to_bf16_bits(r), wl.f32_to_bf16_bits(g)
    assert np.array_equal(oracle.rmsnorm(rb, gb, eps),
                          oracle.rmsnorm(oracle.to_double(rb), oracle.to_double(gb), eps))


def test_block_with_zero_down_weight_is_residual_plus_bias():
    inp = wl.random_inputs(6, 4, 32, 48, wl.BF16, with_down=True)
    r = inp["x"]
    gamma = wl.f32_to_bf16_bits(np.linspace(0.5, 1.5, 32).astype(np.float32))
    wd0 = np.zeros_like(inp["wd"])
    bias = wl.f32_to_bf16_bits(np.linspace(-1, 1, 32).astype(np.float32))
    out = oracle.mlp_block(r, gamma, 1e-5, inp["wg"], inp["wu"], wd0, bias=bias)
    assert np.array_equal(out, oracle.to_double(r) + oracle.to_double(bias)[None, :])
    assert np.array_equal(oracle.mlp_block(r, gamma, 1e-5, inp["wg"], inp["wu"], wd0),
                          oracle.to_double(r))


def test_block_on_unit_rms_rows_is_residual_plus_mlp():
    # rows of +-1 have mean square 1: with gamma = 1 and eps = 0 the norm is
    # the identity, so the block is r + mlp(r) with the pinned MLP
    rng = np.random.default_rng(8)
    M, d, dff = 3, 32, 40
    r = wl.f32_to_bf16_bits(rng.choice([-1.0, 1.0], (M, d)).astype(np.float32))
    one = wl.f32_to_bf16_bits(np.ones(d, dtype=np.float32))
    inp = wl.random_inputs(9, M, d, dff, wl.BF16, with_down=True)
    got = oracle.mlp_block(r, one, 0.0, inp["wg"], inp["wu"], inp["wd"])
    want = oracle.to_double(r) + oracle.mlp(r, inp["wg"], inp["wu"], inp["wd"])
    assert np.allclose(got, want, rtol=1e-14, atol=1e-14)
    rows = [2, 0]
    assert np.array_equal(oracle.mlp_block(r, one, 0.0, inp["wg"], inp["wu"], inp["wd"], rows=rows),
                          got[rows])
