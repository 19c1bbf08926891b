"""Edge sizes through the C ABI against the oracle: the largest M, d and
d_ff the library accepts (2^18 rows, a 2^20 contraction, 2^20 output
columns), the smallest shapes (d = d_ff = 8), for every dtype; the large
cases compare sampled rows or every output the oracle finishes quickly."""
import numpy as np
import pytest

import gemv_gate_up_amd as sw
import oracle
import workloads as wl
from swiglu_testlib import assert_close, dev, host, pack, run_mlp, run_up, say

pytestmark = pytest.mark.gpu

BF16, F32, W8, W4 = wl.BF16, wl.F32, wl.FP8W, wl.MXFP4W
MAX_M, MAX_DIM = 1 << 18, 1 << 20


def _ref_up(inp, dtype, rows=None):
    x, wg, wu = inp["x"], inp["wg"], inp["wu"]
    if dtype == W8:
        return oracle.swiglu_fp8w(x, *oracle.quantize_e4m3(wg), *oracle.quantize_e4m3(wu),
                                  rows=rows)
    if dtype == W4:
        return oracle.swiglu(oracle.to_double(x), oracle.dequantize_mxfp4(*oracle.quantize_mxfp4(wg)),
                             oracle.dequantize_mxfp4(*oracle.quantize_mxfp4(wu)), rows=rows)
    return oracle.swiglu(x, wg, wu, rows=rows)


@pytest.mark.parametrize("path", [sw.SWIGLU_PATH_AUTO, sw.SWIGLU_PATH_SKINNY])
def test_largest_batch(path):
    M, d, dff = MAX_M, 64, 64
    say("max M", M, "path", path)
    inp = wl.random_inputs(101, M, d, dff, BF16, with_down=True)
    wp, wdp = pack(inp, d, dff, BF16)
    out = run_up(dev(inp["x"]), wp, M, d, dff, BF16, path)
    rows = [0, 1, 63, 64, 4097, M // 2 + 5, M - 65, M - 1]
    assert_close(host(out[rows], BF16), oracle.swiglu(inp["x"], inp["wg"], inp["wu"], rows=rows),
                 BF16, "max M up")
    y = run_mlp(dev(inp["x"]), wp, wdp, M, d, dff, BF16, path)
    assert_close(host(y[rows], BF16), oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"],
                                                 rows=rows), BF16, "max M mlp")


@pytest.mark.parametrize("dtype", [BF16, F32, W8, W4])
def test_longest_contraction(dtype):
    M, d, dff = 3, MAX_DIM, 24
    say("max d", dtype)
    inp = wl.random_inputs(102, M, d, dff, dtype)
    wp, _ = pack(inp, d, dff, dtype)
    out = host(run_up(dev(inp["x"]), wp, M, d, dff, dtype), dtype)
    assert_close(out, _ref_up(inp, dtype), dtype, "max d")
    if dtype == BF16:   # the wide kernel too: a 2^20-long K loop through scalar offsets
        out = host(run_up(dev(inp["x"]), wp, M, d, dff, dtype, sw.SWIGLU_PATH_WIDE), dtype)
        assert_close(out, _ref_up(inp, dtype), dtype, "max d wide")


@pytest.mark.parametrize("dtype", [BF16, F32, W8, W4])
def test_widest_output(dtype):
    M, d, dff = 2, 64, MAX_DIM
    say("max dff", dtype)
    inp = wl.random_inputs(103, M, d, dff, dtype)
    wp, _ = pack(inp, d, dff, dtype)
    out = host(run_up(dev(inp["x"]), wp, M, d, dff, dtype), dtype)
    assert_close(out, _ref_up(inp, dtype), dtype, "max dff")


@pytest.mark.parametrize("dtype", [BF16, F32, W8, W4])
def test_smallest_shapes(dtype):
    d = dff = 8
    for M in (1, 3):
        inp = wl.random_inputs(104 + M, M, d, dff, dtype, with_down=True)
        wp, wdp = pack(inp, d, dff, dtype)
        out = host(run_up(dev(inp["x"]), wp, M, d, dff, dtype), dtype)
        assert_close(out, _ref_up(inp, dtype), dtype, "min up M=%d" % M)
        if dtype in (BF16, F32):
            y = host(run_mlp(dev(inp["x"]), wp, wdp, M, d, dff, dtype), dtype)
            assert_close(y, oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"]), dtype,
                         "min mlp M=%d" % M)


def test_limits_are_enforced():
    assert sw.swiglu_packed_bytes(MAX_DIM + 8, 64, BF16) == 0
    assert sw.swiglu_packed_bytes(64, MAX_DIM + 8, BF16) == 0
    assert sw.swiglu_workspace_bytes(MAX_M + 1, 64, 64, BF16, 0) == 0
