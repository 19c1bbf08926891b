"""Row-major activations whose K is padded by a whole chunk (d = 32 mod 64
for bf16).

The packed bf16 weights hold an even number of 32-K chunks, so at such a d
the last chunk of every K loop lies past the activations' K.  On the
row-major plan (x read in place; the block's normalised rows in the
workspace) the lanes of that chunk must read zeros: reading on would take
the next row's first values, and for the last row bytes past the end of the
activations, and multiply them by the weights' zero padding, where an Inf
or a NaN would still turn a finite output into NaN.  Each case poisons what
follows the activations with NaN (or Inf) and requires finite outputs equal
bit for bit to the packed plan's, which never reads past K, and within the
bf16 tolerance of the oracle."""
import numpy as np
import pytest

import oracle
import workloads as wl
from swiglu_testlib import assert_close, bytes_buf, dev, empty, host, pack, say, torch_mod

BF16 = wl.BF16
NAN_BF16, INF_BF16 = 0x7FC0, 0x7F80

pytestmark = pytest.mark.gpu


def sw_mod():
    import gemv_gate_up_amd as sw
    return sw


def _poisoned_x(x: np.ndarray, poison: int):
    """x (M x d bf16 bits) on the device, followed in the same allocation by
    one row and 64 more elements of `poison`."""
    M, d = x.shape
    buf = np.full((M + 1) * d + 64, poison, dtype=np.uint16)
    buf[:M * d] = x.reshape(-1)
    return dev(buf)


@pytest.mark.parametrize("poison", [NAN_BF16, INF_BF16])
@pytest.mark.parametrize("path", ["WIDE", "WIDE_PHASED"])
@pytest.mark.parametrize("shape", [(300, 288, 712), (64 + 33, 96, 520), (256, 4128, 1024)])
def test_up_row_major_reads_nothing_past_k(shape, path, poison):
    sw = sw_mod()
    torch = torch_mod()
    M, d, dff = shape
    assert d % 64 == 32
    say("k-tail up", shape, path, hex(poison))
    p = getattr(sw, "SWIGLU_PATH_" + path)
    inp = wl.random_inputs(71 + M, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    xbuf = _poisoned_x(inp["x"], poison)
    nb = sw.swiglu_workspace_bytes_ex(M, d, dff, BF16, 0, p)
    packed = empty((M, dff), BF16)
    in_place = empty((M, dff), BF16)
    sw.check(sw.swiglu_up_ex(xbuf, wp, packed, M, d, dff, BF16, bytes_buf(nb), nb, None, p))
    sw.check(sw.swiglu_up_ex(xbuf, wp, in_place, M, d, dff, BF16, None, 0, None, p))
    torch.cuda.synchronize()
    got = host(in_place, BF16)
    assert np.all(np.isfinite(got)), "row-major plan read past K"
    assert torch.equal(packed, in_place)
    rows = [0, 1, M // 2, M - 2, M - 1]
    assert_close(got[rows], oracle.swiglu(inp["x"], inp["wg"], inp["wu"], rows=rows), BF16,
                 "k-tail up %s" % (shape,))


@pytest.mark.parametrize("shape", [(300, 288, 712), (130, 96, 1400)])
def test_mlp_row_major_reads_nothing_past_k(shape):
    sw = sw_mod()
    torch = torch_mod()
    M, d, dff = shape
    say("k-tail mlp", shape)
    inp = wl.random_inputs(81 + M, M, d, dff, BF16, with_down=True)
    wp, wdp = pack(inp, d, dff, BF16)
    xbuf = _poisoned_x(inp["x"], NAN_BF16)
    nb = sw.swiglu_workspace_bytes_ex(M, d, dff, BF16, 1, sw.SWIGLU_PATH_WIDE)
    ws = bytes_buf(nb)
    a = empty((M, d), BF16)
    b = empty((M, d), BF16)
    sw.check(sw.mlp_forward_ex(xbuf, wp, wdp, a, M, d, dff, BF16, ws, nb, None,
                               sw.SWIGLU_PATH_WIDE))
    ws.fill_(0xFF)   # NaN wherever the row-major plan might read stale bytes
    sw.check(sw.mlp_forward_ex(xbuf, wp, wdp, b, M, d, dff, BF16, ws, nb - 1, None,
                               sw.SWIGLU_PATH_WIDE))
    torch.cuda.synchronize()
    got = host(b, BF16)
    assert np.all(np.isfinite(got))
    assert torch.equal(a, b)
    rows = [0, M // 2, M - 1]
    assert_close(got[rows], oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"], rows=rows),
                 BF16, "k-tail mlp %s" % (shape,))


def test_block_row_major_reads_nothing_past_k():
    # the block's row-major plan keeps the normalised rows n (lda = d) in
    # the workspace, followed by h: the bytes after the last row of n are
    # NaN-filled workspace when the gate/up product reads n
    sw = sw_mod()
    torch = torch_mod()
    M, d, dff = 130, 288, 712
    say("k-tail block", M, d, dff)
    inp = wl.random_inputs(91, M, d, dff, BF16, with_down=True)
    wp, wdp = pack(inp, d, dff, BF16)
    r = dev(inp["x"])
    gamma = dev(wl.to_storage(1.0 + 0.1 * wl.normal(9, (d,), 1.0), BF16))
    nb = sw.mlp_block_workspace_bytes_ex(M, d, dff, BF16, sw.SWIGLU_PATH_WIDE)
    ws = bytes_buf(nb)
    a = empty((M, d), BF16)
    b = empty((M, d), BF16)
    sw.check(sw.mlp_block_forward_ex(r, gamma, 1e-6, wp, wdp, None, a, M, d, dff, BF16, ws, nb,
                                     None, sw.SWIGLU_PATH_WIDE))
    ws.fill_(0xFF)
    sw.check(sw.mlp_block_forward_ex(r, gamma, 1e-6, wp, wdp, None, b, M, d, dff, BF16, ws,
                                     nb - 1, None, sw.SWIGLU_PATH_WIDE))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(host(b, BF16)))
    assert torch.equal(a, b)
