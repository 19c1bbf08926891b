"""Plant typical mistakes in copies of the oracle's C source (on the CPU)
and check that the pins reject every one of them, while accepting the real
oracle.  This shows the pins are sharp enough to catch a dropped term, a
wrong sign, a transposed operand, a wrong index or a swapped pairing."""
import os

import numpy as np
import pytest
import scipy.special

import oracle
import workloads as wl

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "sigmoid_sign": ("return z * oracle_sigmoid(z);", "return z * oracle_sigmoid(-z);"),
    "swapped_pairing": ("h[r * dff + n] = oracle_silu(gv) * uv;",
                        "h[r * dff + n] = oracle_silu(uv) * gv;"),
    "dropped_first_term": ("for (int64_t k = 0; k < d; ++k) {",
                           "for (int64_t k = 1; k < d; ++k) {"),
    "transposed_gate": ("gs[n - n0] += xv * elem(wg, dtype, k * dff + n);",
                        "gs[n - n0] += xv * elem(wg, dtype, n * d + k);"),
    "transposed_x": ("double xv = elem(x, dtype, m * d + k);",
                     "double xv = elem(x, dtype, k * M + m);"),
    "transposed_down": ("y[r * d + j] += hv * elem(wd, dtype, n * d + j);",
                        "y[r * d + j] += hv * elem(wd, dtype, j * dff + n);"),
    "bf16_shift": ("uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    "up_uses_gate": ("us[n - n0] += xv * elem(wu, dtype, k * dff + n);",
                     "us[n - n0] += xv * elem(wg, dtype, k * dff + n);"),
    "dropped_last_down_term": ("for (int64_t n = 0; n < dff; ++n) {\n                    double hv",
                               "for (int64_t n = 0; n < dff - 1; ++n) {\n                    double hv"),
    # FP8 weight format and quantiser
    "e4m3_bias": ("ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 11)"),
    "e4m3_subnormal_step": ("double v = e == 0 ? ldexp((double)m, -9)",
                            "double v = e == 0 ? ldexp((double)m, -10)"),
    "e4m3_ties_away": ("nearbyint(a / spacing)", "round(a / spacing)"),
    "e4m3_no_saturation": ("if (a >= 448.0)\n        return sign | 0x7E;",
                           "if (a >= 480.0)\n        return sign | 0x7E;"),
    "scale_wrong_max": ("float s = amax / 448.0f;", "float s = amax / 240.0f;"),
    "quantize_unscaled": ("oracle_e4m3_from_float(x / s)", "oracle_e4m3_from_float(x)"),
    "dequantize_unscaled": ("out[k * N + n] = (double)scales[n] * oracle_e4m3_to_double",
                            "out[k * N + n] = oracle_e4m3_to_double"),
    "f64_read_as_f32": ("return ((const double *)p)[i];",
                        "return (double)((const float *)p)[i];"),
    # MXFP4
    "e2m1_bias": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e - 2)"),
    "e2m1_ties_away": ("nearbyint(a / step) * step", "round(a / step) * step"),
    "mx_exponent_offset": ("int s = (e - 1) - 2;", "int s = (e - 1) - 3;"),
    "mx_zero_block": ("    if (amax == 0.0 || isnan(amax))\n        return 0;",
                      "    if (amax == 0.0 || isnan(amax))\n        return -126;"),
    "mx_unscaled_codes": ("oracle_e2m1_from_double(ldexp(oracle_bf16_to_double(w[k * N + n]), -s))",
                          "oracle_e2m1_from_double(oracle_bf16_to_double(w[k * N + n]))"),
    "mx_first_block_scale": ("(int)scales[(k / 32) * N + n] - 127", "(int)scales[n] - 127"),
    # RMSNorm
    "rms_no_eps": ("sqrt(ss / (double)d + eps)", "sqrt(ss / (double)d)"),
    "rms_sum_not_mean": ("sqrt(ss / (double)d + eps)", "sqrt(ss + eps)"),
    "rms_no_sqrt": ("1.0 / sqrt(ss / (double)d + eps)", "1.0 / (ss / (double)d + eps)"),
    "rms_no_gain": ("out[m * d + i] = elem(r, dtype, m * d + i) * inv * elem(gamma, dtype, i);",
                    "out[m * d + i] = elem(r, dtype, m * d + i) * inv;"),
}


def _dec(a):
    return a.astype(np.float64) if a.dtype == np.float32 else wl.bf16_bits_to_f32(a).astype(np.float64)


def pin_failures(lib):
    """Run a compact set of the pins against `lib`; return the failed ones."""
    failed = []

    def check(name, fn):
        try:
            if not fn():
                failed.append(name)
        except Exception:  # a crash or a raised error counts as a failure
            failed.append(name)

    check("bf16", lambda: oracle.bf16_to_double(0x4049, lib=lib) == 3.140625)
    # E4M3 values and codes fixed by the format (worked by hand: 0.3 lies in
    # [2^-2, 2^-1), spacing 2^-5, 9.6 steps -> 10 -> 1.25 * 2^-2 = code 0x2A)
    check("e4m3_decode", lambda: [oracle.e4m3_to_double(c, lib=lib) for c in (0x01, 0x08, 0x38, 0x7E)]
          == [2.0 ** -9, 2.0 ** -6, 1.0, 448.0])
    enc = [(1.0625, 0x38), (1.1875, 0x3A), (3 * 2.0 ** -10, 0x02), (7.5 * 2.0 ** -9, 0x08),
           (475.0, 0x7E), (-1e9, 0xFE), (5.5, 0x4B), (0.3, 0x2A)]
    check("e4m3_encode", lambda: all(oracle.e4m3_from_float(v, lib=lib) == c for v, c in enc))

    def quant_grid():
        col = np.array([448.0, -1.0, 0.5, 3 * 2.0 ** -9], dtype=np.float32) * np.float32(0.25)
        q, sc = oracle.quantize_e4m3(wl.f32_to_bf16_bits(col.reshape(4, 1)), lib=lib)
        return sc[0] == 0.25 and list(q[:, 0]) == [0x7E, 0xB8, 0x30, 0x03]

    check("quantize_grid", quant_grid)
    check("dequantize", lambda: np.array_equal(
        oracle.dequantize_e4m3(np.array([[0x7E], [0xB8]], dtype=np.uint8),
                               np.array([0.25], dtype=np.float32), lib=lib),
        np.array([[112.0], [-0.25]])))

    def f64_path():
        inp = wl.random_inputs(12, 2, 16, 8, wl.BF16)
        f = {k: wl.bf16_bits_to_f32(v).astype(np.float64) for k, v in inp.items()}
        return np.array_equal(oracle.swiglu(f["x"], f["wg"], f["wu"], lib=lib),
                              oracle.swiglu(inp["x"], inp["wg"], inp["wu"], lib=lib))

    check("f64_path", f64_path)
    # MXFP4: E2M1 values, ties, the shared exponent, a two-block exact grid
    check("e2m1", lambda: [oracle.e2m1_to_double(c, lib=lib) for c in (1, 5, 7)] == [0.5, 3.0, 6.0]
          and [oracle.e2m1_from_double(v, lib=lib) for v in (0.75, 2.5, 5.0)] == [2, 4, 6])
    check("mx_exp", lambda: [oracle.mx_shared_exponent(a, lib=lib) for a in (1.0, 6.0, 0.0)]
          == [-2, 0, 0])

    def mx_grid():
        col = np.array([6.0, -0.5, 1.5] + [0.0] * 29 + [4.0, 3.0, -1.0], dtype=np.float32)
        col[:32] *= np.float32(2.0 ** -3)
        col[32:] *= np.float32(2.0 ** 2)
        q, sc = oracle.quantize_mxfp4(wl.f32_to_bf16_bits(col.reshape(-1, 1)), lib=lib)
        deq = oracle.dequantize_mxfp4(q, sc, lib=lib)[:, 0]
        return (list(sc[:, 0]) == [124, 129] and list(q[[0, 1, 2, 32, 33, 34], 0]) == [7, 9, 3, 6, 5, 10]
                and np.array_equal(deq, col.astype(np.float64)))

    check("mx_grid", mx_grid)
    # RMSNorm: the hand-worked row [3, 4] (n = [0.6, 0.8] * sqrt 2), a gain,
    # and the eps closed form at d = 1
    check("rmsnorm_hand", lambda: np.allclose(
        oracle.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0, lib=lib)[0],
        [0.6 * np.sqrt(2), 1.6 * np.sqrt(2)], rtol=1e-15, atol=0))
    check("rmsnorm_eps", lambda: abs(
        oracle.rmsnorm(np.array([[0.3]]), np.array([1.0]), 1e-2, lib=lib)[0, 0]
        - 0.3 / np.sqrt(0.09 + 1e-2)) < 1e-15)
    check("silu_log3", lambda: abs(oracle.silu(np.log(3.0), lib=lib) - np.log(3.0) * 0.75) < 1e-15)
    for dtype in (wl.F32, wl.BF16):
        inp = wl.integer_inputs(5, 3, 37, 29, dtype, with_down=True, lo=-3, hi=3)
        xi = _dec(inp["x"]).astype(np.int64)
        gi = (xi @ _dec(inp["wg"]).astype(np.int64)).astype(np.float64)
        ui = (xi @ _dec(inp["wu"]).astype(np.int64)).astype(np.float64)
        href = gi * scipy.special.expit(gi) * ui
        yref = href @ _dec(inp["wd"])

        def prod():
            _, g, u = oracle.swiglu(inp["x"], inp["wg"], inp["wu"], want_gu=True, lib=lib)
            return np.array_equal(g, gi) and np.array_equal(u, ui)

        def act():
            h = oracle.swiglu(inp["x"], inp["wg"], inp["wu"], lib=lib)
            return np.allclose(h, href, rtol=1e-14, atol=0)

        def down():
            y = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"], lib=lib)
            return np.allclose(y, yref, rtol=1e-12, atol=1e-12)

        check("products_%d" % dtype, prod)
        check("activation_%d" % dtype, act)
        check("down_%d" % dtype, down)
    return failed


def test_real_oracle_passes_compact_pins():
    assert pin_failures(None) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, "mutation anchor not found: " + name
    mut = tmp_path / ("oracle_%s.c" % name)
    mut.write_text(src.replace(before, after))
    lib = oracle.load_library(oracle.compile_source(str(mut), str(tmp_path / ("lib%s.so" % name))))
    assert pin_failures(lib), "planted mistake %s went unnoticed" % name
