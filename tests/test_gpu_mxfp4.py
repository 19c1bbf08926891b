"""MXFP4-weight path (SWIGLU_BF16_MXFP4W) through the C ABI: packed E2M1
codes and E8M0 block scales must equal the oracle's quantiser bit for bit
(every rounding decision is exact on both sides), and the products must
match the oracle's fp64 product of x with the same dequantised weights."""
import numpy as np
import pytest

import gemv_gate_up_amd as sw
import oracle
import workloads as wl
from swiglu_testlib import (assert_close, bytes_buf, dev, host, pack, run_mlp, run_up, say,
                            torch_mod)

pytestmark = pytest.mark.gpu

W4 = wl.MXFP4W


def unpack_mxfp4(buf: np.ndarray, K: int, ncols: int, plain: bool):
    """Host reading of the MXFP4 packed layout: pieces [pair block][128-K
    piece][half][k-group][column][chunk j][byte i] with two codes per byte
    (low nibble first), then block scales [pair block][piece][half][column]
    [chunk].  Returns codes (K_pad x cols) and scales (K_pad/32 x cols) per
    matrix: gate and up for the fused buffer, one matrix for down."""
    nkc = -(-K // 128)
    npb = -(-(-(-ncols // (32 if plain else 16))) // 8) * 8
    nb = npb * nkc * 2 * 1024
    assert buf.size == nb + npb * nkc * 2 * 64
    by = buf[:nb].reshape(npb, nkc, 2, 4, 16, 4, 4)            # pb kc h g c j i
    nib = np.stack([by & 15, by >> 4], axis=-1)                  # ... i nib
    sc = buf[nb:].reshape(npb, nkc, 2, 16, 4)                    # pb kc h c j
    if plain:
        codes = nib.transpose(1, 5, 3, 6, 7, 0, 2, 4).reshape(nkc * 128, npb * 32)
        return codes, sc.transpose(1, 4, 0, 2, 3).reshape(nkc * 4, npb * 32)
    codes = nib.transpose(2, 1, 5, 3, 6, 7, 0, 4).reshape(2, nkc * 128, npb * 16)
    scales = sc.transpose(2, 1, 4, 0, 3).reshape(2, nkc * 4, npb * 16)
    return (codes[0], scales[0]), (codes[1], scales[1])


@pytest.mark.parametrize("d,dff", [(128, 16), (136, 40), (520, 1048), (4096, 264), (1000, 24)])
def test_pack_matches_the_oracle_quantiser_bitwise(d, dff):
    say("mxfp4 pack", d, dff)
    inp = wl.random_inputs(d + 3 * dff, 1, d, dff, W4, with_down=True)
    inp["wg"][:, 3] = 0                          # all-zero blocks
    inp["wu"][:40, 5] = 0
    inp["wu"][7, 1] = wl.f32_to_bf16_bits(np.array([50.0], dtype=np.float32))[0]
    # non-finite weights: NaN and infinities are coded +-6, a NaN does not
    # count toward its block's exponent (also in an otherwise zero block),
    # an infinity puts it at the top
    inp["wg"][2, 4] = 0x7FC0
    inp["wu"][:, 7] = 0
    inp["wu"][3, 7] = 0xFFC0
    inp["wg"][40, 6] = 0xFF80
    inp["wd"][5, 2] = 0x7F80
    wp, wdp = pack(inp, d, dff, W4)
    (qg, sg), (qu, su) = unpack_mxfp4(wp.cpu().numpy(), d, dff, plain=False)
    nbk = -(-d // 32)
    for (q, s), w in (((qg, sg), inp["wg"]), ((qu, su), inp["wu"])):
        rq, rs = oracle.quantize_mxfp4(w)
        assert np.array_equal(q[:d, :dff], rq)
        assert np.array_equal(s[:nbk, :dff], rs)
        assert not q[d:].any() and not q[:, dff:].any()
        assert np.all(s[nbk:] == 127) and np.all(s[:, dff:] == 127)
    qd, sd = unpack_mxfp4(wdp.cpu().numpy(), dff, d, plain=True)
    rq, rs = oracle.quantize_mxfp4(inp["wd"])
    assert np.array_equal(qd[:dff, :d], rq)
    assert np.array_equal(sd[:-(-dff // 32), :d], rs)


def _deq(inp):
    return {k: oracle.dequantize_mxfp4(*oracle.quantize_mxfp4(inp[k]))
            for k in ("wg", "wu", "wd") if k in inp}


# (40, 520, 8200) and (64, 1032, 8200): four pair blocks per workgroup at
# 17-64 rows, ragged tail; (6, 264, 8192): one workgroup per CU on eight waves
@pytest.mark.parametrize("shape", [(1, 512, 2048), (3, 264, 200), (16, 1032, 776),
                                   (17, 520, 1048), (40, 136, 3000), (64, 896, 4864),
                                   (100, 328, 1000), (40, 520, 8200), (64, 1032, 8200),
                                   (6, 264, 8192)])
def test_up_mxfp4_random(shape):
    M, d, dff = shape
    say("up mxfp4", shape)
    inp = wl.random_inputs(M * 13 + d, M, d, dff, W4)
    wp, _ = pack(inp, d, dff, W4)
    out = host(run_up(dev(inp["x"]), wp, M, d, dff, W4), W4)
    w = _deq(inp)
    ref = oracle.swiglu(oracle.to_double(inp["x"]), w["wg"], w["wu"])
    assert_close(out, ref, W4, "up mxfp4 %s" % (shape,))


@pytest.mark.parametrize("shape", [(1, 256, 512), (7, 136, 392), (64, 896, 4864),
                                   (130, 264, 712)])
def test_mlp_mxfp4_random(shape):
    M, d, dff = shape
    say("mlp mxfp4", shape)
    inp = wl.random_inputs(M + 7 * d, M, d, dff, W4, with_down=True)
    wp, wdp = pack(inp, d, dff, W4)
    y = host(run_mlp(dev(inp["x"]), wp, wdp, M, d, dff, W4), W4)
    w = _deq(inp)
    ref = oracle.mlp(oracle.to_double(inp["x"]), w["wg"], w["wu"], w["wd"])
    assert_close(y, ref, W4, "mlp mxfp4 %s" % (shape,))


def test_exact_grid_weights_give_exact_products():
    # power-of-two multiples of E2M1 values with a +-4 or +-6 per block
    # quantise exactly; with small integer x every partial sum is exact in
    # fp32, so only silu and the bf16 rounding remain
    rng = np.random.default_rng(10)
    M, d, dff = 8, 512, 272
    x = rng.integers(-3, 4, (M, d)).astype(np.float32)
    table = np.array([oracle.e2m1_to_double(c) for c in range(16)])

    def grid(n):
        c = rng.integers(0, 16, (d, n))
        for b in range(d // 32):
            c[32 * b + rng.integers(0, 32), np.arange(n)] = rng.choice([6, 7, 14, 15], n)
        s = np.repeat(rng.integers(-8, -3, (d // 32, n)), 32, axis=0)
        return (table[c] * np.exp2(s)).astype(np.float32)

    wg, wu = grid(dff), grid(dff)
    inp = {"x": wl.f32_to_bf16_bits(x), "wg": wl.f32_to_bf16_bits(wg),
           "wu": wl.f32_to_bf16_bits(wu)}
    wp, _ = pack(inp, d, dff, W4)
    out = host(run_up(dev(inp["x"]), wp, M, d, dff, W4), W4)
    ref = oracle.swiglu(x.astype(np.float64), wg.astype(np.float64), wu.astype(np.float64))
    assert np.all(np.abs(out - ref) <= (2.0 ** -8 + 1e-5) * np.abs(ref) + 1e-30)


def test_mxfp4_split_path_and_refused_wide_paths():
    M, d, dff = 1, 16384, 512
    assert sw.swiglu_workspace_bytes(M, d, dff, W4, 0) > 0
    inp = wl.random_inputs(78, M, d, dff, W4)
    wp, _ = pack(inp, d, dff, W4)
    out = bytes_buf(M * dff * 2)
    for path in (sw.SWIGLU_PATH_WIDE, sw.SWIGLU_PATH_WIDE_PHASED):
        assert sw.swiglu_up_ex(dev(inp["x"]), wp, out, M, d, dff, W4, None, 0, None,
                               path) == sw.SWIGLU_ERR_UNSUPPORTED
    a = run_up(dev(inp["x"]), wp, M, d, dff, W4)
    b = run_up(dev(inp["x"]), wp, M, d, dff, W4).cpu().numpy()
    assert np.array_equal(a.cpu().numpy(), b)
    w = _deq(inp)
    assert_close(host(a, W4), oracle.swiglu(oracle.to_double(inp["x"]), w["wg"], w["wu"]), W4,
                 "split")
    torch_mod().cuda.synchronize()
