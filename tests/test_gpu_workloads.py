"""GPU parity at the full workload sizes, in the launch configuration the
bench times (automatic path), against the oracle: every output where the
oracle finishes in seconds, else whole sampled rows spread over tiles and
the ragged last tile."""
import numpy as np
import torch  # noqa: F401  (first import on a fresh box is slow; keep it out of test timeouts)
import pytest

import oracle
import workloads as wl
from swiglu_testlib import assert_close, dev, host, pack, run_mlp, run_up, say

pytestmark = pytest.mark.gpu

_cache = {}


def _inputs(name):
    w = wl.WORKLOADS[name]
    key = (w.cfg, w.with_down)
    if key not in _cache:
        _cache.clear()
        full = wl.WORKLOADS[name]
        inp = wl.make_inputs(full, M=full.m_max)
        wp, wdp = pack(inp, w.d, w.dff, w.dtype)
        _cache[key] = (inp, wp, wdp)
    return _cache[key]


def _rows(M):
    """All rows up to 64; else whole rows spread over the output: one in every
    256-row tile (a different offset in each), the first and last rows of
    the last (possibly ragged) tile, and the rows next to the 128-row and
    256-row tile boundaries."""
    if M <= 64:
        return None                    # all rows
    cand = [0, 1, 127, 128, 255, 256, M // 2 + 3, M - 257, M - 2, M - 1]
    cand += [t * 256 + (t * 37 + 11) % 256 for t in range(-(-M // 256))]
    cand += [(M - 1) // 256 * 256]
    return sorted({r for r in cand if 0 <= r < M})


@pytest.mark.parametrize("name", ["tiny_decode_f32", "decode8b_m1", "decode8b_m4", "decode8b_m8",
                                  "decode8b_m16", "prefill8b_m4096", "prefill8b_m128",
                                  "prefill8b_m256", "prefill8b_m512", "up72b_m512"])
def test_up_workload(name):
    w = wl.WORKLOADS[name]
    say("workload", name, w)
    inp, wp, _ = _inputs(name)
    x = inp["x"][:w.M]
    out = run_up(dev(x), wp, w.M, w.d, w.dff, w.dtype)
    rows = _rows(w.M)
    got = host(out if rows is None else out[rows], w.dtype)
    ref = oracle.swiglu(x, inp["wg"], inp["wu"], rows=rows)
    st = assert_close(got, ref, w.dtype, name)
    say(name, st)


@pytest.mark.parametrize("name", ["mlp05b_m64", "mlp72b_m16", "mlp72b_m2048"])
def test_mlp_workload(name):
    w = wl.WORKLOADS[name]
    say("workload", name, w)
    inp, wp, wdp = _inputs(name)
    x = inp["x"][:w.M]
    y = run_mlp(dev(x), wp, wdp, w.M, w.d, w.dff, w.dtype)
    rows = _rows(w.M)
    got = host(y if rows is None else y[rows], w.dtype)
    ref = oracle.mlp(x, inp["wg"], inp["wu"], inp["wd"], rows=rows)
    st = assert_close(got, ref, w.dtype, name)
    say(name, st)


@pytest.mark.parametrize("name", ["decode8b_m1_mxfp4w", "decode8b_m16_mxfp4w", "mlp72b_m16_mxfp4w"])
def test_mxfp4w_workload(name):
    # MXFP4 weights at the decode shapes against the oracle's product with
    # its own quantisation of the same bf16 weights (the packer's codes and
    # scales equal it bit for bit: test_gpu_mxfp4.py)
    w = wl.WORKLOADS[name]
    say("workload", name, w)
    inp = wl.make_inputs(w, M=w.M)
    wp, wdp = pack(inp, w.d, w.dff, w.dtype)
    deq = {k: oracle.dequantize_mxfp4(*oracle.quantize_mxfp4(inp[k]))
           for k in ("wg", "wu", "wd") if k in inp}
    x64 = oracle.to_double(inp["x"])
    if w.with_down:
        out = run_mlp(dev(inp["x"]), wp, wdp, w.M, w.d, w.dff, w.dtype)
        ref = oracle.mlp(x64, deq["wg"], deq["wu"], deq["wd"])
    else:
        out = run_up(dev(inp["x"]), wp, w.M, w.d, w.dff, w.dtype)
        ref = oracle.swiglu(x64, deq["wg"], deq["wu"])
    st = assert_close(host(out, w.dtype), ref, w.dtype, name)
    say(name, st)


@pytest.mark.parametrize("name", ["decode8b_m1_fp8w", "decode8b_m16_fp8w", "mlp72b_m16_fp8w"])
def test_fp8w_workload(name):
    # FP8 weights at the decode shapes: reference = the oracle's product with
    # the oracle's own quantisation of the same bf16 weights (the packer's
    # codes equal it bit for bit: test_gpu_fp8w.py)
    w = wl.WORKLOADS[name]
    say("workload", name, w)
    inp = wl.make_inputs(w, M=w.M)
    wp, wdp = pack(inp, w.d, w.dff, w.dtype)
    q = {k: oracle.quantize_e4m3(inp[k]) for k in ("wg", "wu", "wd") if k in inp}
    if w.with_down:
        out = run_mlp(dev(inp["x"]), wp, wdp, w.M, w.d, w.dff, w.dtype)
        ref = oracle.mlp_fp8w(inp["x"], *q["wg"], *q["wu"], *q["wd"])
    else:
        out = run_up(dev(inp["x"]), wp, w.M, w.d, w.dff, w.dtype)
        ref = oracle.swiglu_fp8w(inp["x"], *q["wg"], *q["wu"])
    st = assert_close(host(out, w.dtype), ref, w.dtype, name)
    say(name, st)


def test_mlp72b_tensor_parallel_shard():
    # One GPU's share of the 72B-class MLP split eight ways over d_ff
    # (29568 / 8 = 3696 columns, not a multiple of the 128-column tile).
    d, dff = 8192, 3696
    for M in (16, 300):
        say("tp shard", M, d, dff)
        inp = wl.random_inputs(5000 + M, M, d, dff, wl.BF16, with_down=True)
        wp, wdp = pack(inp, d, dff, wl.BF16)
        y = host(run_mlp(dev(inp["x"]), wp, wdp, M, d, dff, wl.BF16), wl.BF16)
        rows = _rows(M)
        ref = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"], rows=rows)
        assert_close(y if rows is None else y[rows], ref, wl.BF16, "tp shard M=%d" % M)
