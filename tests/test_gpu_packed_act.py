"""The many-rows path with and without the packed activation layout.

With the workspace that swiglu_workspace_bytes reports, the MFMA GEMM reads
its left operand in the packed layout (x packed into the workspace, h
written packed by the gate/up kernel, RMSNorm's rows written packed); with a
smaller workspace that still holds the row-major plan it reads the same
values in place.  Both run the same MFMAs in the same order, so the results
must agree bit for bit; the parity tests compare the packed plan with the
oracle.  Shapes with a ragged last row block, K not a whole number of
chunks, and dff not a whole number of tiles."""
import numpy as np
import pytest

import workloads as wl
from swiglu_testlib import bytes_buf, dev, empty, pack, say, torch_mod

BF16 = wl.BF16

pytestmark = pytest.mark.gpu

SHAPES = [(130, 264, 712), (256, 512, 1408), (77, 1024, 2816), (300, 4096, 1024)]


def sw_mod():
    import gemv_gate_up_amd as sw
    return sw


@pytest.mark.parametrize("path", ["WIDE", "WIDE_PHASED"])
@pytest.mark.parametrize("shape", SHAPES)
def test_up_packed_and_in_place_agree(shape, path):
    sw = sw_mod()
    M, d, dff = shape
    say("packed/in-place up", shape, path)
    p = getattr(sw, "SWIGLU_PATH_" + path)
    inp = wl.random_inputs(11 + M, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    x = dev(inp["x"])
    nb = sw.swiglu_workspace_bytes_ex(M, d, dff, BF16, 0, p)
    assert nb == -(-M // 16) * -(-d // 64) * 2 * 1024
    ws = bytes_buf(nb)
    a = empty((M, dff), BF16)
    b = empty((M, dff), BF16)
    sw.check(sw.swiglu_up_ex(x, wp, a, M, d, dff, BF16, ws, nb, None, p))
    sw.check(sw.swiglu_up_ex(x, wp, b, M, d, dff, BF16, None, 0, None, p))
    torch_mod().cuda.synchronize()
    assert torch_mod().equal(a, b)


@pytest.mark.parametrize("shape", SHAPES)
def test_mlp_packed_and_in_place_agree(shape):
    sw = sw_mod()
    M, d, dff = shape
    say("packed/in-place mlp", shape)
    inp = wl.random_inputs(21 + M, M, d, dff, BF16, with_down=True)
    wp, wdp = pack(inp, d, dff, BF16)
    x = dev(inp["x"])
    nb = sw.swiglu_workspace_bytes_ex(M, d, dff, BF16, 1, sw.SWIGLU_PATH_WIDE)
    ws = bytes_buf(nb)
    a = empty((M, d), BF16)
    b = empty((M, d), BF16)
    sw.check(sw.mlp_forward_ex(x, wp, wdp, a, M, d, dff, BF16, ws, nb, None, sw.SWIGLU_PATH_WIDE))
    # one byte short of the packed plan: the row-major plan (h row-major in
    # the same workspace, x read in place)
    sw.check(sw.mlp_forward_ex(x, wp, wdp, b, M, d, dff, BF16, ws, nb - 1, None,
                               sw.SWIGLU_PATH_WIDE))
    torch_mod().cuda.synchronize()
    assert torch_mod().equal(a, b)


# rows not a multiple of 16: the packed rows take more room than the
# row-major ones, so one byte less selects the row-major plan (with every
# size aligned the two plans need the same workspace)
@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[2]])
def test_block_packed_and_in_place_agree(shape):
    sw = sw_mod()
    M, d, dff = shape
    say("packed/in-place block", shape)
    inp = wl.random_inputs(31 + M, M, d, dff, BF16, with_down=True)
    wp, wdp = pack(inp, d, dff, BF16)
    r = dev(inp["x"])
    gamma = dev(wl.to_storage(1.0 + 0.1 * wl.normal(7, (d,), 1.0), BF16))
    nb = sw.mlp_block_workspace_bytes_ex(M, d, dff, BF16, sw.SWIGLU_PATH_WIDE)
    ws = bytes_buf(nb)
    a = empty((M, d), BF16)
    b = empty((M, d), BF16)
    sw.check(sw.mlp_block_forward_ex(r, gamma, 1e-6, wp, wdp, None, a, M, d, dff, BF16, ws, nb,
                                     None, sw.SWIGLU_PATH_WIDE))
    sw.check(sw.mlp_block_forward_ex(r, gamma, 1e-6, wp, wdp, None, b, M, d, dff, BF16, ws,
                                     nb - 1, None, sw.SWIGLU_PATH_WIDE))
    torch_mod().cuda.synchronize()
    assert torch_mod().equal(a, b)


def test_too_small_workspace_is_still_rejected():
    # both products of this shape take the wide path (108 and 50 workgroups
    # at 300 rows), whose packed plan needs more than the row-major h; every
    # plan of an MLP needs at least that h, so less is rejected before any
    # launch (the weights here are placeholders of 16 bytes)
    sw = sw_mod()
    M, d, dff = 300, 3080, 3400
    assert sw.swiglu_select_path(M, d, dff, BF16) == sw.SWIGLU_PATH_WIDE
    nb = sw.swiglu_workspace_bytes(M, d, dff, BF16, 1)
    row_major_h = M * (-(-dff // 128) * 128) * 2
    assert nb > row_major_h
    rc = sw.mlp_forward(dev(np.zeros((M, d), np.uint16)), bytes_buf(16), bytes_buf(16),
                        empty((M, d), BF16), M, d, dff, BF16, bytes_buf(row_major_h - 256),
                        row_major_h - 256, stream=0)
    assert rc == sw.SWIGLU_ERR_WORKSPACE
