"""Seeded random shapes on the many-rows path (M from 65 up, d and dff any
multiple of 8): partial row tiles, K not a whole number of chunks, dff not a
whole number of pair blocks or tiles.  On each shape the packed-operand
plan, the in-place plan and the two-pass schedule must agree bit for bit,
and sampled rows must match the oracle; likewise for the full MLP."""
import numpy as np
import pytest

import oracle
import workloads as wl
from swiglu_testlib import (assert_close, bytes_buf, dev, empty, host, pack, run_mlp, say,
                            torch_mod)

pytestmark = pytest.mark.gpu

BF16 = wl.BF16
_rng = np.random.default_rng(20261202)
UP_SHAPES = [(int(_rng.integers(65, 1100)), 8 * int(_rng.integers(8, 300)),
              8 * int(_rng.integers(8, 700))) for _ in range(12)]
MLP_SHAPES = [(int(_rng.integers(65, 700)), 8 * int(_rng.integers(8, 200)),
               8 * int(_rng.integers(8, 400))) for _ in range(6)]


def _rows(M):
    return sorted({0, 15, 16, M // 2, M - 1})


@pytest.mark.parametrize("shape", UP_SHAPES, ids=[str(s) for s in UP_SHAPES])
def test_random_up_shape(shape):
    import gemv_gate_up_amd as sw
    M, d, dff = shape
    say("random up shape", shape)
    inp = wl.random_inputs(M + d + dff, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    x = dev(inp["x"])
    outs = []
    for path, packed in ((sw.SWIGLU_PATH_WIDE, True), (sw.SWIGLU_PATH_WIDE, False),
                         (sw.SWIGLU_PATH_WIDE_PHASED, True)):
        nb = sw.swiglu_workspace_bytes_ex(M, d, dff, BF16, 0, path) if packed else 0
        ws = bytes_buf(nb) if nb else None
        out = empty((M, dff), BF16)
        sw.check(sw.swiglu_up_ex(x, wp, out, M, d, dff, BF16, ws, nb, None, path))
        outs.append(out)
    torch_mod().cuda.synchronize()
    assert torch_mod().equal(outs[0], outs[1]), "packed and in-place plans differ"
    assert torch_mod().equal(outs[0], outs[2]), "one-pass and two-pass schedules differ"
    rows = _rows(M)
    ref = oracle.swiglu(inp["x"], inp["wg"], inp["wu"], rows=rows)
    assert_close(host(outs[0][rows], BF16), ref, BF16, "random up %s" % (shape,))


@pytest.mark.parametrize("shape", MLP_SHAPES, ids=[str(s) for s in MLP_SHAPES])
def test_random_mlp_shape(shape):
    import gemv_gate_up_amd as sw
    M, d, dff = shape
    say("random mlp shape", shape)
    inp = wl.random_inputs(M + d + dff + 1, M, d, dff, BF16, with_down=True)
    wp, wdp = pack(inp, d, dff, BF16)
    x = dev(inp["x"])
    nb = sw.swiglu_workspace_bytes_ex(M, d, dff, BF16, 1, sw.SWIGLU_PATH_WIDE)
    ws = bytes_buf(nb)
    a = empty((M, d), BF16)
    b = empty((M, d), BF16)
    sw.check(sw.mlp_forward_ex(x, wp, wdp, a, M, d, dff, BF16, ws, nb, None, sw.SWIGLU_PATH_WIDE))
    sw.check(sw.mlp_forward_ex(x, wp, wdp, b, M, d, dff, BF16, ws, nb - 1, None,
                               sw.SWIGLU_PATH_WIDE))
    torch_mod().cuda.synchronize()
    assert torch_mod().equal(a, b), "packed and row-major plans differ"
    rows = _rows(M)
    ref = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"], rows=rows)
    assert_close(host(a[rows], BF16), ref, BF16, "random mlp %s" % (shape,))
