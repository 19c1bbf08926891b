"""Non-finite activations through the C ABI: plain IEEE propagation, no
special handling.  One row of x holds a NaN and another an infinity.  The
oracle (fp64, the same IEEE rules) must put NaN and infinities in exactly
the same outputs, with the same signs, as the GPU.  Every other row must
stay finite and within tolerance, which also shows that no kernel mixes
rows (a wrong row index or a missing mask would spread the poison)."""
import numpy as np
import pytest

import gemv_gate_up_amd as sw
import oracle
import workloads as wl
from swiglu_testlib import assert_close, dev, host, pack, run_mlp, run_up, say

pytestmark = pytest.mark.gpu

BF16, F32, W8, W4 = wl.BF16, wl.F32, wl.FP8W, wl.MXFP4W
AUTO, SKINNY, WIDE = sw.SWIGLU_PATH_AUTO, sw.SWIGLU_PATH_SKINNY, sw.SWIGLU_PATH_WIDE
NAN_ROW, INF_ROW = 1, 2


def _poisoned(seed, M, d, dff, dtype, with_down=False):
    inp = wl.random_inputs(seed, M, d, dff, dtype, with_down=with_down)
    x = inp["x"].copy()
    if dtype == F32:
        x[NAN_ROW, 7] = np.nan
        x[INF_ROW, d - 5] = np.inf
    else:
        x[NAN_ROW, 7] = 0x7FC0          # bf16 NaN
        x[INF_ROW, d - 5] = 0x7F80      # bf16 +inf
    inp["x"] = x
    return inp


def _check(got, ref, dtype, what):
    assert np.array_equal(np.isnan(got), np.isnan(ref)), what + ": NaN positions"
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf), what + ": infinity positions"
    assert np.array_equal(np.sign(got[inf]), np.sign(ref[inf])), what + ": infinity signs"
    # the poisoned rows are entirely non-finite here, the others entirely finite
    assert not np.isfinite(ref[NAN_ROW]).any() and not np.isfinite(ref[INF_ROW]).any(), what
    clean = [r for r in range(ref.shape[0]) if r not in (NAN_ROW, INF_ROW)]
    assert np.isfinite(ref[clean]).all(), what
    assert_close(got[clean], ref[clean], dtype, what)


def _ref_up(inp, dtype):
    x, wg, wu = inp["x"], inp["wg"], inp["wu"]
    if dtype == W8:
        return oracle.swiglu_fp8w(x, *oracle.quantize_e4m3(wg), *oracle.quantize_e4m3(wu))
    if dtype == W4:
        return oracle.swiglu(oracle.to_double(x), oracle.dequantize_mxfp4(*oracle.quantize_mxfp4(wg)),
                             oracle.dequantize_mxfp4(*oracle.quantize_mxfp4(wu)))
    return oracle.swiglu(x, wg, wu)


# (M, d, dff, dtype, path): few rows on the skinny kernel, with and without
# a split of K; many rows on the wide kernel; fp32; FP8 and MXFP4 weights
UP_CASES = [(4, 512, 1024, BF16, SKINNY), (3, 4096, 512, BF16, SKINNY),
            (200, 512, 1024, BF16, WIDE), (5, 512, 512, F32, AUTO),
            (4, 512, 1024, W8, AUTO), (4, 512, 1024, W4, AUTO)]


@pytest.mark.parametrize("case", UP_CASES)
def test_up_propagates_nan_and_inf_within_their_rows(case):
    M, d, dff, dtype, path = case
    say("non-finite up", case)
    inp = _poisoned(6100 + M, M, d, dff, dtype)
    wp, _ = pack(inp, d, dff, dtype)
    got = host(run_up(dev(inp["x"]), wp, M, d, dff, dtype, path), dtype)
    _check(got, _ref_up(inp, dtype), BF16 if dtype in (W8, W4) else dtype, "up %s" % (case,))


@pytest.mark.parametrize("case", [(16, 768, 1280, BF16, SKINNY), (300, 512, 1024, BF16, WIDE),
                                  (4, 256, 512, F32, AUTO)])
def test_mlp_propagates_nan_and_inf_within_their_rows(case):
    M, d, dff, dtype, path = case
    say("non-finite mlp", case)
    inp = _poisoned(6200 + M, M, d, dff, dtype, with_down=True)
    wp, wdp = pack(inp, d, dff, dtype)
    got = host(run_mlp(dev(inp["x"]), wp, wdp, M, d, dff, dtype, path), dtype)
    _check(got, oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"]), dtype, "mlp %s" % (case,))
