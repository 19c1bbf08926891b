"""The fused down projection (SWIGLU_PATH_FUSED_DOWN) through the C ABI.

Each workgroup forms a slice of h in LDS and writes that slice's share of y;
a second pass adds the slices in order.  Checked against the oracle's fp64
MLP on every element: at the full 0.5B-class shape (M = 64, d = 896,
d_ff = 4864) and the 72B-class decode shape (M = 16), and on ragged shapes
(rows not a multiple of 16, more than one row group, d_ff not a whole number
of slices, d not a whole number of 32-column blocks); bitwise determinism;
the MLP block (RMSNorm, bias, residual) on the same path; and the other
paths' results within the bf16 bar."""
import numpy as np
import pytest

import oracle
import workloads as wl
from swiglu_testlib import (assert_close, bytes_buf, dev, empty, host, pack, run_mlp, say,
                            torch_mod)

BF16 = wl.BF16
pytestmark = pytest.mark.gpu


def sw_mod():
    import gemv_gate_up_amd as sw
    return sw


def fused(x, wp, wdp, M, d, dff):
    sw = sw_mod()
    return run_mlp(x, wp, wdp, M, d, dff, BF16, path=sw.SWIGLU_PATH_FUSED_DOWN)


@pytest.mark.parametrize("name", ["mlp05b_m64", "mlp72b_m16"])
def test_fused_workload_every_element(name):
    torch = torch_mod()
    w = wl.WORKLOADS[name]
    say("fused workload", name)
    inp = wl.make_inputs(w, M=w.M)
    wp, wdp = pack(inp, w.d, w.dff, BF16)
    x = dev(inp["x"])
    y = fused(x, wp, wdp, w.M, w.d, w.dff)
    st = assert_close(host(y, BF16), oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"]), BF16,
                      name + " fused")
    say(name, st)
    # bitwise determinism: a second call gives the same bits
    y2 = fused(x, wp, wdp, w.M, w.d, w.dff)
    assert torch.equal(y, y2)


SHAPES = [(1, 256, 512), (7, 136, 392), (16, 1032, 776), (17, 264, 712), (33, 520, 1400),
          (48, 96, 4880), (64, 896, 4864), (100, 512, 1400), (16, 8192, 3696)]


@pytest.mark.parametrize("shape", SHAPES)
def test_fused_shapes(shape):
    M, d, dff = shape
    say("fused shape", shape)
    inp = wl.random_inputs(4100 + M + d, M, d, dff, BF16, with_down=True)
    wp, wdp = pack(inp, d, dff, BF16)
    x = dev(inp["x"])
    y = host(fused(x, wp, wdp, M, d, dff), BF16)
    ref = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"])
    assert_close(y, ref, BF16, "fused %s" % (shape,))
    # the unfused paths agree within the same bar
    sk = host(run_mlp(x, wp, wdp, M, d, dff, BF16), BF16)
    assert_close(y, sk, BF16, "fused vs automatic %s" % (shape,))


def test_fused_integer_exact():
    # small-integer inputs: g and u are exact in fp32 whatever the order, h
    # is rounded once to bf16 as on the other paths; with one-hot down
    # columns y picks single values of that rounded h (the GPU's fp32 silu
    # and the oracle's fp64 one may round to neighbouring bf16 values: one
    # ulp, 2^-7 relative)
    M, d, dff = 20, 128, 256
    x = wl.to_storage(wl.small_int(11, (M, d), -2, 2), BF16)
    wg = wl.to_storage(wl.small_int(12, (d, dff), -2, 2), BF16)
    wu = wl.to_storage(wl.small_int(13, (d, dff), -2, 2), BF16)
    pick = np.arange(d) * 2 % dff
    wd = np.zeros((dff, d), dtype=np.float32)
    wd[pick, np.arange(d)] = 1.0
    inp = {"x": x, "wg": wg, "wu": wu, "wd": wl.to_storage(wd, BF16)}
    wp, wdp = pack(inp, d, dff, BF16)
    y = host(fused(dev(x), wp, wdp, M, d, dff), BF16)
    h = oracle.swiglu(x, wg, wu)
    h_bf16 = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(h.astype(np.float32))).astype(np.float64)
    np.testing.assert_allclose(y, h_bf16[:, pick], rtol=2.0 ** -7, atol=0)


def test_fused_block_bias_and_residual():
    sw = sw_mod()
    torch = torch_mod()
    M, d, dff = 40, 896, 4864
    say("fused block", M, d, dff)
    inp = wl.random_inputs(4200, M, d, dff, BF16, with_down=True)
    rng = np.random.default_rng(4200)
    r = wl.to_storage((wl.normal(4201, (M, d), 1.0) *
                       rng.uniform(0.25, 4.0, (M, 1))).astype(np.float32), BF16)
    gamma = wl.to_storage(1.0 + 0.2 * rng.standard_normal(d).astype(np.float32), BF16)
    bias = wl.to_storage(0.1 * rng.standard_normal(d).astype(np.float32), BF16)
    wp, wdp = pack(inp, d, dff, BF16)
    path = sw.SWIGLU_PATH_FUSED_DOWN
    nb = sw.mlp_block_workspace_bytes_ex(M, d, dff, BF16, path)
    ws = bytes_buf(nb)
    out = empty((M, d), BF16)
    sw.check(sw.mlp_block_forward_ex(dev(r), dev(gamma), 1e-6, wp, wdp, dev(bias), out, M, d,
                                     dff, BF16, ws, nb, None, path))
    torch.cuda.synchronize()
    ref = oracle.mlp_block(r, gamma, 1e-6, inp["wg"], inp["wu"], inp["wd"], bias=bias)
    assert_close(host(out, BF16), ref, BF16, "fused block")
    # in place: out = r
    rr = dev(r)
    sw.check(sw.mlp_block_forward_ex(rr, dev(gamma), 1e-6, wp, wdp, dev(bias), rr, M, d, dff,
                                     BF16, ws, nb, None, path))
    torch.cuda.synchronize()
    assert torch.equal(rr, out)
