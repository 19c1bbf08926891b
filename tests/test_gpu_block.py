"""The MLP half of a layer through the C ABI (mlp_block_forward): RMSNorm
prologue, SwiGLU MLP, bias and residual epilogue, against the oracle's fp64
block on the skinny, split-K, wide and FP8-weight paths; plus exact
residual/bias arithmetic and the in-place residual update."""
import numpy as np
import pytest

import gemv_gate_up_amd as sw
import oracle
import workloads as wl
from swiglu_testlib import assert_close, bytes_buf, dev, empty, host, pack, say, torch_mod

pytestmark = pytest.mark.gpu

BF16, F32, W8, W4 = wl.BF16, wl.F32, wl.FP8W, wl.MXFP4W
EPS = 1e-6


def _block_inputs(seed, M, d, dff, dtype):
    inp = wl.random_inputs(seed, M, d, dff, dtype, with_down=True)
    rng = np.random.default_rng(seed)
    sto = lambda a: wl.to_storage(a.astype(np.float32), dtype)
    # rows of different scales, so the normalisation matters
    r = wl.normal(seed * 16 + 7, (M, d), 1.0) * rng.uniform(0.25, 4.0, (M, 1)).astype(np.float32)
    inp["r"] = sto(r)
    inp["gamma"] = sto(1.0 + 0.2 * rng.standard_normal(d))
    inp["bias"] = sto(0.1 * rng.standard_normal(d))
    return inp


def _run(inp, wp, wdp, M, d, dff, dtype, bias=True, path=0, inplace=False):
    nb = sw.mlp_block_workspace_bytes_ex(M, d, dff, dtype, path)
    ws = bytes_buf(nb)
    r = dev(inp["r"])
    out = r if inplace else empty((M, d), dtype)
    b = dev(inp["bias"]) if bias else None
    sw.check(sw.mlp_block_forward_ex(r, dev(inp["gamma"]), EPS, wp, wdp, b, out, M, d, dff,
                                     dtype, ws, nb, None, path), "mlp_block_forward_ex")
    torch_mod().cuda.synchronize()
    return out


def _reference(inp, dtype, bias=True):
    w = {k: inp[k] for k in ("wg", "wu", "wd")}
    if dtype == W8:
        w = {k: oracle.dequantize_e4m3(*oracle.quantize_e4m3(v)) for k, v in w.items()}
    if dtype == W4:
        w = {k: oracle.dequantize_mxfp4(*oracle.quantize_mxfp4(v)) for k, v in w.items()}
    return oracle.mlp_block(inp["r"], inp["gamma"], EPS, w["wg"], w["wu"], w["wd"],
                            bias=inp["bias"] if bias else None)


CASES = [
    (1, 256, 512, BF16, 0), (7, 136, 392, BF16, 0), (64, 896, 4864, BF16, 0),
    (130, 264, 712, BF16, 0), (300, 1000, 1400, BF16, 0), (96, 512, 1408, BF16, 1),
    (130, 264, 712, BF16, 2), (300, 1000, 1400, BF16, 2),
    (4, 100, 60, F32, 0), (12, 64, 520, F32, 0),
    (16, 1032, 776, W8, 0), (64, 896, 4864, W8, 0),
    (16, 1032, 776, W4, 0), (64, 896, 4864, W4, 0),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("bias", [True, False])
def test_block_matches_oracle(case, bias):
    M, d, dff, dtype, path = case
    say("block", case, "bias", bias)
    inp = _block_inputs(M + d + dff, M, d, dff, dtype)
    wp, wdp = pack(inp, d, dff, dtype)
    out = host(_run(inp, wp, wdp, M, d, dff, dtype, bias, path), dtype)
    assert_close(out, _reference(inp, dtype, bias), dtype, "block %s" % (case,))


@pytest.mark.parametrize("case", [(16, 1024, 1408, BF16, 0), (300, 1000, 1400, BF16, 0),
                                  (300, 1000, 1400, BF16, 2), (1, 512, 2048, F32, 0),
                                  (16, 1032, 776, W8, 0)])
def test_block_in_place_equals_out_of_place(case):
    M, d, dff, dtype, path = case
    inp = _block_inputs(3 * M + d, M, d, dff, dtype)
    wp, wdp = pack(inp, d, dff, dtype)
    a = _run(inp, wp, wdp, M, d, dff, dtype, path=path).cpu().numpy()
    b = _run(inp, wp, wdp, M, d, dff, dtype, path=path, inplace=True).cpu().numpy()
    assert np.array_equal(a, b)


# (M, d, dff, path): besides the small case, two wide-path down products
# whose residual epilogue runs in 256 x 256 tiles with ragged rows and
# columns (9 x 17 tiles), and in 7 rounds of them plus quarter tiles for the
# last (9 x 30 tiles)
ZERO_DOWN = [(80, 256, 384, sw.SWIGLU_PATH_SKINNY), (80, 256, 384, sw.SWIGLU_PATH_WIDE),
             (2100, 4104, 256, sw.SWIGLU_PATH_WIDE), (2100, 7560, 256, sw.SWIGLU_PATH_WIDE)]


@pytest.mark.parametrize("case", ZERO_DOWN)
@pytest.mark.parametrize("bias", [True, False])
def test_zero_down_weight_gives_rounded_residual_plus_bias(case, bias):
    # h . 0 = 0 exactly, so out = round(0 + r + bias); with bf16 r and bias
    # the fp32 sum is exact here, so the result is the nearest bf16 of it.
    # The products' sum starts from +0, so a residual of -0 (a bf16 draw
    # that rounds to it) gives +0 without a bias (IEEE: +0 + -0 = +0).
    M, d, dff, path = case
    say("zero down", case, "bias", bias)
    inp = _block_inputs(11, M, d, dff, BF16)
    inp["wd"] = np.zeros_like(inp["wd"])
    wp, wdp = pack(inp, d, dff, BF16)
    out = _run(inp, wp, wdp, M, d, dff, BF16, bias, path).cpu().numpy().view(np.uint16)
    want = 0.0 + wl.bf16_bits_to_f32(inp["r"]).astype(np.float64)
    if bias:
        want = want + wl.bf16_bits_to_f32(inp["bias"]).astype(np.float64)
    want = wl.f32_to_bf16_bits(want.astype(np.float32))
    bad = np.argwhere(out != want)
    assert bad.size == 0, "%d mismatches, rows %s, columns %s, first %s: %s != %s" % (
        len(bad), np.unique(bad[:, 0])[:12], np.unique(bad[:, 1])[:12], bad[:4].tolist(),
        wl.bf16_bits_to_f32(out[tuple(bad[:4].T)]), wl.bf16_bits_to_f32(want[tuple(bad[:4].T)]))


# The down product on 256 x 256 tiles (9 x 17 of them, ragged rows and
# columns), and on 7 rounds of them plus quarter tiles for the last (9 x 30):
# the tile's products are staged in LDS a quarter at a time and the bias and
# residual added as the rows are written; sampled rows cover every quarter.
@pytest.mark.parametrize("shape", [(2100, 4104, 1024), (2100, 7560, 512)])
@pytest.mark.parametrize("bias", [True, False])
def test_block_on_full_tiles_against_the_oracle(shape, bias):
    M, d, dff = shape
    say("block full tiles", shape, "bias", bias)
    inp = _block_inputs(5 + M + d, M, d, dff, BF16)
    wp, wdp = pack(inp, d, dff, BF16)
    out = host(_run(inp, wp, wdp, M, d, dff, BF16, bias, sw.SWIGLU_PATH_WIDE), BF16)
    rows = sorted({0, 63, 64, 127, 128, 191, 192, 255, 256, 1791, 1792, 2047, 2048, M - 1}
                  | set(range(5, M, 89)))
    ref = oracle.mlp_block(inp["r"], inp["gamma"], EPS, inp["wg"], inp["wu"], inp["wd"],
                           bias=inp["bias"] if bias else None, rows=rows)
    say(assert_close(out[rows], ref, BF16, "block full tiles %s" % (shape,)))
