"""The wide path's last partial round of 256 x 256 tiles runs as quarter
tiles in a second launch (when it would occupy at most half the compute
units).  Every output still sums the same MFMAs in the same K order, so the
gate/up product must equal the two-pass schedule (which never splits its
tail) bit for bit; both products are also checked against the oracle on
rows that cross the quarter tiles, including a partial last row tile whose
lower quarter tiles fall outside the output."""
import numpy as np
import pytest

import oracle
import workloads as wl
from swiglu_testlib import assert_close, dev, empty, host, pack, run_mlp, run_up, say, torch_mod

pytestmark = pytest.mark.gpu

BF16 = wl.BF16

# (M, d, dff): 256 x 256 tile grids of 260 (4 tail tiles), 2 x 130 = 260
# with a 44-row last tile row, and 356 (100 tail tiles)
UP_SHAPES = [(256, 256, 33280), (300, 128, 16640), (256, 128, 45568)]


def _rows(M):
    return sorted({0, 1, 127, 128, 129, 255, M - 1} | {r for r in range(3, M, 37)})


@pytest.mark.parametrize("shape", UP_SHAPES)
def test_gateup_tail_matches_the_unsplit_schedule(shape):
    import gemv_gate_up_amd as sw
    M, d, dff = shape
    say("tail gate/up", shape)
    inp = wl.random_inputs(41 + M, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    x = dev(inp["x"])
    split = run_up(x, wp, M, d, dff, BF16, sw.SWIGLU_PATH_WIDE)
    plain = run_up(x, wp, M, d, dff, BF16, sw.SWIGLU_PATH_WIDE_PHASED)
    assert torch_mod().equal(split, plain)
    rows = _rows(M)
    ref = oracle.swiglu(inp["x"], inp["wg"], inp["wu"], rows=rows)
    say(assert_close(host(split[rows], BF16), ref, BF16, "tail gate/up %s" % (shape,)))


def test_down_tail_against_the_oracle():
    # down product: 33 x 8 = 264 tiles of 256 x 256 (8 tail tiles); the
    # gate/up product has 66 tiles and no tail
    M, d, dff = 8448, 2048, 256
    say("tail down", (M, d, dff))
    inp = wl.random_inputs(47, M, d, dff, BF16, with_down=True)
    wp, wdp = pack(inp, d, dff, BF16)
    y = run_mlp(dev(inp["x"]), wp, wdp, M, d, dff, BF16)
    rows = sorted({0, 255, 2304, 2559, M - 256, M - 1} | {r for r in range(5, M, 61)})
    ref = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"], rows=rows)
    say(assert_close(host(y[rows], BF16), ref, BF16, "tail down"))
