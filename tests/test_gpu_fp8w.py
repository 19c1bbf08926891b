"""FP8-weight path (SWIGLU_BF16_FP8W) through the C ABI: the packer's codes
and column scales must equal the oracle's quantiser bit for bit (both take
their rounding decisions in fp32), and the products must match the oracle's
fp64 product of x with the same dequantised weights."""
import numpy as np
import pytest

import gemv_gate_up_amd as sw
import oracle
import workloads as wl
from swiglu_testlib import (assert_close, bytes_buf, dev, host, pack, run_mlp, run_up, say,
                            torch_mod)

pytestmark = pytest.mark.gpu

W8 = wl.FP8W


def _geom(K, ncols, cols_per_pb):
    nkc = -(-K // 64)
    npb = -(-(-(-ncols // cols_per_pb)) // 8) * 8
    return nkc, npb


def unpack_fp8(buf: np.ndarray, K: int, ncols: int, plain: bool):
    """Host reading of the FP8 packed layout: pieces [pair block][64-K chunk]
    [half][k-group][column][2 x 8 codes], then fp32 scales [pair block][half]
    [16].  Returns (codes K_pad x cols, scales cols) per matrix: gate and up
    for the fused buffer, one matrix for the down buffer."""
    nkc, npb = _geom(K, ncols, 32 if plain else 16)
    nb = npb * nkc * 2 * 1024
    assert buf.size == nb + npb * 32 * 4
    arr = buf[:nb].reshape(npb, nkc, 2, 4, 16, 2, 8)      # pb kc h g c j e
    scales = buf[nb:].view(np.float32).reshape(npb, 2, 16)
    if plain:
        codes = arr.transpose(1, 5, 3, 6, 0, 2, 4).reshape(nkc * 64, npb * 32)
        return codes, scales.reshape(npb * 32)
    codes = arr.transpose(2, 1, 5, 3, 6, 0, 4).reshape(2, nkc * 64, npb * 16)
    return (codes[0], scales[:, 0].reshape(-1)), (codes[1], scales[:, 1].reshape(-1))


PACK_SHAPES = [(64, 16), (104, 40), (520, 1048), (4096, 264), (1000, 24)]


@pytest.mark.parametrize("d,dff", PACK_SHAPES)
def test_pack_matches_the_oracle_quantiser_bitwise(d, dff):
    say("fp8 pack", d, dff)
    inp = wl.random_inputs(d + dff, 1, d, dff, W8, with_down=True)
    # columns the quantiser must treat specially: all zero, one spike
    inp["wg"][:, 3] = 0
    inp["wu"][:, 5] = 0
    inp["wu"][7, 1] = wl.f32_to_bf16_bits(np.array([50.0], dtype=np.float32))[0]
    # non-finite weights: a NaN (code 0x7F, no effect on the scale), a NaN in
    # an otherwise zero column (scale 0, code 0), -inf (infinite scale)
    inp["wg"][2, 4] = 0x7FC0
    inp["wu"][:, 7] = 0
    inp["wu"][3, 7] = 0x7FC0
    inp["wg"][9, 6] = 0xFF80
    inp["wd"][5, 2] = 0x7FC0
    wp, wdp = pack(inp, d, dff, W8)
    buf = wp.cpu().numpy()
    (qg, sg), (qu, su) = unpack_fp8(buf, d, dff, plain=False)
    for (q, s), w in (((qg, sg), inp["wg"]), ((qu, su), inp["wu"])):
        rq, rs = oracle.quantize_e4m3(w)
        assert np.array_equal(q[:d, :dff], rq)
        assert np.array_equal(s[:dff].view(np.uint32), rs.view(np.uint32))
        assert not q[d:].any() and not q[:, dff:].any() and not s[dff:].any()
    qd, sd = unpack_fp8(wdp.cpu().numpy(), dff, d, plain=True)
    rq, rs = oracle.quantize_e4m3(inp["wd"])
    assert np.array_equal(qd[:dff, :d], rq)
    assert np.array_equal(sd[:d].view(np.uint32), rs.view(np.uint32))


# (40, 520, 8200): four pair blocks per workgroup at 17-64 rows, ragged tail;
# (16, 264, 18944): 1,184 pair blocks, two per workgroup for balance;
# (5, 264, 8192): 512 pair blocks, one workgroup per CU on eight waves
UP_SHAPES = [(1, 512, 2048), (3, 264, 200), (16, 1032, 776), (17, 520, 1048), (40, 136, 3000),
             (64, 896, 4864), (100, 328, 1000), (40, 520, 8200), (16, 264, 18944), (5, 264, 8192)]


def _quantised(inp):
    return {k: oracle.quantize_e4m3(inp[k]) for k in ("wg", "wu", "wd") if k in inp}


@pytest.mark.parametrize("shape", UP_SHAPES)
def test_up_fp8w_random(shape):
    M, d, dff = shape
    say("up fp8w", shape)
    inp = wl.random_inputs(M * 11 + d, M, d, dff, W8)
    wp, _ = pack(inp, d, dff, W8)
    out = host(run_up(dev(inp["x"]), wp, M, d, dff, W8), W8)
    q = _quantised(inp)
    ref = oracle.swiglu_fp8w(inp["x"], *q["wg"], *q["wu"])
    assert_close(out, ref, W8, "up fp8w %s" % (shape,))


@pytest.mark.parametrize("shape", [(1, 256, 512), (7, 136, 392), (64, 896, 4864), (130, 264, 712)])
def test_mlp_fp8w_random(shape):
    M, d, dff = shape
    say("mlp fp8w", shape)
    inp = wl.random_inputs(M + 5 * d, M, d, dff, W8, with_down=True)
    wp, wdp = pack(inp, d, dff, W8)
    y = host(run_mlp(dev(inp["x"]), wp, wdp, M, d, dff, W8), W8)
    q = _quantised(inp)
    ref = oracle.mlp_fp8w(inp["x"], *q["wg"], *q["wu"], *q["wd"])
    assert_close(y, ref, W8, "mlp fp8w %s" % (shape,))


def test_exact_grid_weights_give_exact_products():
    # Weights that are power-of-two multiples of E4M3 values with a +-448
    # entry per column quantise exactly; with small integer x every product
    # and partial sum is exact in fp32, so only silu and the final bf16
    # rounding separate the GPU from the oracle.
    rng = np.random.default_rng(9)
    M, d, dff = 8, 640, 272
    codes = [c for c in range(0x70) if c >= 0x38] + [c | 0x80 for c in range(0x38, 0x70)]
    x = rng.integers(-3, 4, (M, d)).astype(np.float32)

    table = np.array([oracle.e4m3_to_double(c) if c not in (0x7F, 0xFF) else 0.0
                      for c in range(256)])

    def grid(n):
        v = table[rng.choice(codes, (d, n))]
        v[rng.integers(0, d, n), np.arange(n)] = 448.0
        return v.astype(np.float32) * np.float32(2.0 ** -12)

    wg, wu = grid(dff), grid(dff)
    inp = {"x": wl.f32_to_bf16_bits(x), "wg": wl.f32_to_bf16_bits(wg),
           "wu": wl.f32_to_bf16_bits(wu)}
    wp, _ = pack(inp, d, dff, W8)
    out = host(run_up(dev(inp["x"]), wp, M, d, dff, W8), W8)
    ref = oracle.swiglu(x.astype(np.float64), wg.astype(np.float64), wu.astype(np.float64))
    bound = (2.0 ** -8 + 1e-5) * np.abs(ref) + 1e-30
    assert np.all(np.abs(out - ref) <= bound)


def test_fp8w_workspace_and_split_path():
    # few output columns over a long K split K across workgroups (partials
    # in the workspace) with FP8 weights too; forced wide paths are refused
    M, d, dff = 1, 4096, 512
    assert sw.swiglu_workspace_bytes(M, d, dff, W8, 0) > 0
    inp = wl.random_inputs(77, M, d, dff, W8)
    wp, _ = pack(inp, d, dff, W8)
    out = bytes_buf(M * dff * 2)
    for path in (sw.SWIGLU_PATH_WIDE, sw.SWIGLU_PATH_WIDE_PHASED):
        assert sw.swiglu_up_ex(dev(inp["x"]), wp, out, M, d, dff, W8, None, 0, None,
                               path) == sw.SWIGLU_ERR_UNSUPPORTED
    a = run_up(dev(inp["x"]), wp, M, d, dff, W8)
    b = run_up(dev(inp["x"]), wp, M, d, dff, W8).cpu().numpy()
    assert np.array_equal(a.cpu().numpy(), b)
    q = _quantised(inp)
    assert_close(host(a, W8), oracle.swiglu_fp8w(inp["x"], *q["wg"], *q["wu"]), W8, "split")
    torch_mod().cuda.synchronize()
