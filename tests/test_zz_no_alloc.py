"""swiglu_up_noalloc through the C ABI: the entry point for callers that
cannot allocate, which keeps its workspace (split-K partials, packed x) in
the library's fixed per-GPU array.  Its output must equal, bit for bit,
swiglu_up's with the workspace swiglu_workspace_bytes reports (the same
kernels in the same order), on two calls in a row, the second with a smaller
input, so that what the first call left in the array cannot leak into the
second; sampled rows are also checked against the oracle."""
import numpy as np
import pytest

import oracle
import workloads as wl
from swiglu_testlib import assert_close, bytes_buf, dev, empty, host, pack, say, torch_mod

pytestmark = pytest.mark.gpu


def sw_mod():
    import gemv_gate_up_amd as sw
    return sw


def _reference_call(sw, x, wp, M, d, dff, dtype):
    nb = sw.swiglu_workspace_bytes(M, d, dff, dtype, 0)
    out = empty((M, dff), dtype)
    sw.check(sw.swiglu_up(x, wp, out, M, d, dff, dtype, bytes_buf(nb) if nb else None, nb),
             "swiglu_up")
    return out, nb


# (label, dtype, d, dff, larger M, smaller M): what each case puts in the array
CASES = [
    # few rows, K split 16 ways: fp32 partials in the array, then the second pass
    ("split-K fp32", wl.F32, 4096, 512, 8, 1),
    # few rows, K split over bf16 pieces (the 16-row tile), partials in the array
    ("split-K bf16", wl.BF16, 8192, 1024, 16, 3),
    # few rows, no split: the array is not touched
    ("decode bf16", wl.BF16, 1024, 2816, 4, 1),
    # many rows: x packed into the array (ragged rows and K; a d_ff whose
    # grid keeps both calls on the wide path)
    ("wide packed x", wl.BF16, 1000, 8200, 300, 97),
    # many rows whose packed x exceeds the array: x read in place
    ("wide in place", wl.BF16, 4096, 512, 4608, 129),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_swiglu_up_on_two_calls(case):
    sw = sw_mod()
    torch = torch_mod()
    label, dtype, d, dff, m_big, m_small = case
    say("noalloc", label, dtype, d, dff, m_big, m_small)
    inp = wl.random_inputs(700 + d % 97, m_big, d, dff, dtype)
    wp, _ = pack(inp, d, dff, dtype)
    x = dev(inp["x"])
    # the workspace the plain call would take, for the record
    nb_big = sw.swiglu_workspace_bytes(m_big, d, dff, dtype, 0)
    if label == "wide in place":
        assert nb_big > sw.SWIGLU_SCRATCH_BYTES
    elif label != "decode bf16":
        assert 0 < nb_big <= sw.SWIGLU_SCRATCH_BYTES
    # two no-alloc calls back to back on one stream, the second smaller
    a_big = empty((m_big, dff), dtype)
    a_small = empty((m_small, dff), dtype)
    sw.check(sw.swiglu_up_noalloc(x, wp, a_big, m_big, d, dff, dtype), "noalloc 1")
    sw.check(sw.swiglu_up_noalloc(x[m_big - m_small:], wp, a_small, m_small, d, dff, dtype),
             "noalloc 2")
    torch.cuda.synchronize()
    r_big, _ = _reference_call(sw, x, wp, m_big, d, dff, dtype)
    r_small, _ = _reference_call(sw, x[m_big - m_small:], wp, m_small, d, dff, dtype)
    torch.cuda.synchronize()
    assert torch.equal(a_big, r_big), label + ": first call differs from swiglu_up"
    assert torch.equal(a_small, r_small), label + ": second call differs from swiglu_up"
    rows = sorted({0, m_big // 2, m_big - 1})
    assert_close(host(a_big, dtype)[rows],
                 oracle.swiglu(inp["x"], inp["wg"], inp["wu"], rows=rows), dtype, label)
    srows = sorted({0, m_small - 1})
    assert_close(host(a_small, dtype)[srows],
                 oracle.swiglu(inp["x"][m_big - m_small:], inp["wg"], inp["wu"], rows=srows),
                 dtype, label + " (second call)")


def test_noalloc_argument_errors_and_no_op():
    sw = sw_mod()
    x = dev(np.zeros((4, 64), np.uint16))
    wp = bytes_buf(sw.swiglu_packed_bytes(64, 64, wl.BF16))
    out = empty((4, 64), wl.BF16)
    assert sw.swiglu_up_noalloc(x, wp, out, -1, 64, 64, wl.BF16) == sw.SWIGLU_ERR_INVALID_ARG
    assert sw.swiglu_up_noalloc(None, wp, out, 4, 64, 64, wl.BF16) == sw.SWIGLU_ERR_INVALID_ARG
    assert sw.swiglu_up_noalloc(x, wp, out, 4, 64, 64, 9) == sw.SWIGLU_ERR_UNSUPPORTED
    assert sw.swiglu_up_noalloc(None, None, None, 0, 64, 64, wl.BF16) == sw.SWIGLU_OK
