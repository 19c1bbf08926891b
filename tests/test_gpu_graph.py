"""Recorded calls (HIP graphs) through the C ABI: every replay must equal
the direct call bit for bit (the same kernels on the same buffers), also
with other GPU work and host synchronisations between replays, after the
input is overwritten in place, and when replayed on another stream."""
import numpy as np
import pytest

import gemv_gate_up_amd as sw
import oracle
import workloads as wl
from swiglu_testlib import assert_close, bytes_buf, dev, empty, host, pack, say, torch_mod

pytestmark = pytest.mark.gpu

BF16, F32 = wl.BF16, wl.F32
AUTO, WIDE, PHASED = sw.SWIGLU_PATH_AUTO, sw.SWIGLU_PATH_WIDE, sw.SWIGLU_PATH_WIDE_PHASED
FUSED = sw.SWIGLU_PATH_FUSED_DOWN

# (M, d, dff, dtype, with_down, path): split-K skinny with its reduce kernel,
# the 4-launch small MLP, the wide kernels, the fp32 skinny path, and the
# fused down projection with its second pass
CASES = [
    (1, 4096, 512, F32, False, AUTO),
    (1, 512, 2048, F32, False, AUTO),
    (64, 896, 4864, BF16, True, AUTO),
    (16, 1024, 1408, BF16, True, AUTO),
    (300, 1000, 1400, BF16, False, WIDE),
    (130, 264, 712, BF16, True, WIDE),
    (257, 520, 2056, BF16, False, PHASED),
    (64, 896, 4864, BF16, True, FUSED),
    (20, 1032, 776, BF16, True, FUSED),
]


def _direct(x, wp, wdp, out, ws, nb, M, d, dff, dtype, with_down, path):
    if with_down:
        return sw.mlp_forward_ex(x, wp, wdp, out, M, d, dff, dtype, ws, nb, None, path)
    return sw.swiglu_up_ex(x, wp, out, M, d, dff, dtype, ws, nb, None, path)


@pytest.mark.parametrize("case", CASES)
def test_graph_replays_equal_the_direct_call(case):
    M, d, dff, dtype, with_down, path = case
    torch = torch_mod()
    say("graph", case)
    inp = wl.random_inputs(71 + M, M, d, dff, dtype, with_down=with_down)
    wp, wdp = pack(inp, d, dff, dtype)
    x = dev(inp["x"])
    ncols = d if with_down else dff
    nb = sw.swiglu_workspace_bytes_ex(M, d, dff, dtype, int(with_down), path)
    ws = bytes_buf(nb)
    out_direct = empty((M, ncols), dtype)
    sw.check(_direct(x, wp, wdp, out_direct, ws, nb, M, d, dff, dtype, with_down, path))
    torch.cuda.synchronize()
    ref = out_direct.clone()

    out = empty((M, ncols), dtype)
    if with_down:
        rc, g = sw.mlp_forward_graph_create(x, wp, wdp, out, M, d, dff, dtype, ws, nb, path)
    else:
        rc, g = sw.swiglu_up_graph_create(x, wp, out, M, d, dff, dtype, ws, nb, path)
    sw.check(rc, "graph create")
    assert g
    try:
        side = torch.cuda.Stream()
        other = torch.randn(512, 512, device="cuda")
        for rep in range(4):
            out.fill_(-1)                     # the replay must rewrite every element
            torch.cuda.synchronize()
            stream = side if rep == 2 else None
            sw.check(sw.swiglu_graph_launch(g, stream), "graph launch")
            torch.cuda.synchronize()
            assert torch.equal(out, ref), "replay %d differs from the direct call" % rep
            # the program's own eager work between replays, sharing the workspace
            other = other @ other.t() * 1e-3
            sw.check(_direct(x, wp, wdp, out_direct, ws, nb, M, d, dff, dtype, with_down, path))
            torch.cuda.synchronize()
        # new input written in place: the replay computes on it
        inp2 = wl.random_inputs(171 + M, M, d, dff, dtype)
        x.copy_(dev(inp2["x"]))
        sw.check(_direct(x, wp, wdp, out_direct, ws, nb, M, d, dff, dtype, with_down, path))
        torch.cuda.synchronize()
        ref2 = out_direct.clone()
        out.fill_(-1)
        sw.check(sw.swiglu_graph_launch(g), "graph launch")
        torch.cuda.synchronize()
        assert torch.equal(out, ref2)
        if with_down:
            expect = oracle.mlp(inp2["x"], inp["wg"], inp["wu"], inp["wd"])
        else:
            expect = oracle.swiglu(inp2["x"], inp["wg"], inp["wu"])
        assert_close(host(out, dtype), expect, dtype, "graph replay on new input")
    finally:
        assert sw.swiglu_graph_destroy(g) == sw.SWIGLU_OK


def test_back_to_back_replays_on_one_stream_run_in_order():
    # ten replays queued without a host wait give the same result as one
    M, d, dff = 64, 896, 4864
    torch = torch_mod()
    inp = wl.random_inputs(5, M, d, dff, BF16, with_down=True)
    wp, wdp = pack(inp, d, dff, BF16)
    x = dev(inp["x"])
    nb = sw.swiglu_workspace_bytes(M, d, dff, BF16, 1)
    ws = bytes_buf(nb)
    out = empty((M, d), BF16)
    rc, g = sw.mlp_forward_graph_create(x, wp, wdp, out, M, d, dff, BF16, ws, nb)
    sw.check(rc)
    try:
        sw.check(sw.swiglu_graph_launch(g))
        torch.cuda.synchronize()
        one = out.clone()
        for _ in range(10):
            sw.check(sw.swiglu_graph_launch(g))
        torch.cuda.synchronize()
        assert torch.equal(out, one)
    finally:
        sw.swiglu_graph_destroy(g)


def test_empty_batch_records_an_empty_graph():
    rc, g = sw.swiglu_up_graph_create(None, None, None, 0, 64, 64, BF16)
    sw.check(rc)
    try:
        sw.check(sw.swiglu_graph_launch(g))
        torch_mod().cuda.synchronize()
    finally:
        sw.swiglu_graph_destroy(g)


# skinny products; skinny products at 130 rows; both products on the wide
# path (300 rows, 108 and 50 workgroups)
@pytest.mark.parametrize("case", [(16, 1024, 1408, BF16), (130, 264, 712, BF16),
                                  (300, 3080, 3400, BF16)])
def test_block_graph_replays_equal_the_direct_call(case):
    M, d, dff, dtype = case
    torch = torch_mod()
    inp = wl.random_inputs(301 + M, M, d, dff, dtype, with_down=True)
    wp, wdp = pack(inp, d, dff, dtype)
    r = dev(inp["x"])
    gamma = dev(wl.to_storage(1.0 + 0.1 * wl.normal(5, (d,), 1.0), dtype))
    bias = dev(wl.to_storage(wl.normal(6, (d,), 0.1), dtype))
    nb = sw.mlp_block_workspace_bytes(M, d, dff, dtype)
    ws = bytes_buf(nb)
    ref = empty((M, d), dtype)
    sw.check(sw.mlp_block_forward(r, gamma, 1e-6, wp, wdp, bias, ref, M, d, dff, dtype, ws, nb))
    torch.cuda.synchronize()
    out = empty((M, d), dtype)
    rc, g = sw.mlp_block_graph_create(r, gamma, 1e-6, wp, wdp, bias, out, M, d, dff, dtype, ws, nb)
    sw.check(rc, "block graph create")
    try:
        for _ in range(3):
            out.fill_(-1)
            torch.cuda.synchronize()
            sw.check(sw.swiglu_graph_launch(g))
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
    finally:
        sw.swiglu_graph_destroy(g)
