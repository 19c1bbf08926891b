"""Calls from several host threads at once.

The header promises thread-safe entry points: the library keeps no mutable
state except launch attributes set once per kernel instantiation and the
no-alloc array's device address, looked up once per device.  Here four
threads start together (a barrier), each on its own stream with its own
output and workspace, and call the library repeatedly; every result must be
bit for bit the one a single thread gets (the kernels are deterministic).
The no-alloc calls share the one array: on a shape that uses none of it
they run concurrently on their own streams (the host side, including the
first-call address lookup, runs at once); on a shape that uses it they
follow the documented rule, one stream and one call at a time."""
import threading

import numpy as np
import pytest

import workloads as wl
from swiglu_testlib import bytes_buf, dev, empty, pack, say, torch_mod

pytestmark = pytest.mark.gpu

BF16, F32, FP8W = wl.BF16, wl.F32, wl.FP8W
THREADS = 4
REPEATS = 6

# (M, d, dff, dtype, with_down): few-rows split-K, a few hundred rows on
# the wide kernel's narrow tiles, many rows on full rounds plus the
# quarter-tile tail (9 x 32 tiles of 256 x 256: one round and 32 tiles),
# the MLP, FP8 weights, fp32
CASES = [
    (1, 1024, 2816, BF16, False),
    (300, 512, 2336, BF16, False),
    (2304, 512, 8192, BF16, False),
    (16, 768, 1280, BF16, True),
    (8, 1024, 1536, FP8W, False),
    (4, 512, 1024, F32, False),
]


def _sw():
    import gemv_gate_up_amd as sw
    return sw


def _call(case, x, wp, wdp, out, ws, nb, stream):
    sw = _sw()
    M, d, dff, dt, down = case
    if down:
        return sw.mlp_forward(x, wp, wdp, out, M, d, dff, dt, ws, nb, stream)
    return sw.swiglu_up(x, wp, out, M, d, dff, dt, ws, nb, stream)


def _prepare(case, seed):
    sw = _sw()
    M, d, dff, dt, down = case
    inp = wl.random_inputs(seed, M, d, dff, dt, with_down=down)
    wp, wdp = pack(inp, d, dff, dt)
    nb = sw.swiglu_workspace_bytes(M, d, dff, dt, 1 if down else 0)
    ocols = d if down else dff
    odt = BF16 if dt == FP8W else dt
    return dev(inp["x"]), wp, wdp, nb, (M, ocols), odt


def _run_threads(work):
    """work: list of callables, one per thread; they start together."""
    gate = threading.Barrier(len(work))
    errors = []

    def body(fn):
        try:
            gate.wait()
            fn()
        except Exception as e:   # reported after the join
            errors.append(e)

    ts = [threading.Thread(target=body, args=(fn,)) for fn in work]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors


def test_threads_own_streams_match_single_thread():
    torch = torch_mod()
    sw = _sw()
    prepared = [_prepare(c, 5100 + i) for i, c in enumerate(CASES)]
    # single-thread references on the default stream
    refs = []
    for case, (x, wp, wdp, nb, shape, odt) in zip(CASES, prepared):
        out = empty(shape, odt)
        ws = bytes_buf(nb)
        sw.check(_call(case, x, wp, wdp, out, ws, nb, None), "reference call")
        refs.append(out)
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in range(THREADS)]
    outs = [[empty(p[4], p[5]) for p in prepared] for _ in range(THREADS)]
    wss = [[bytes_buf(p[3]) for p in prepared] for _ in range(THREADS)]
    status = [[] for _ in range(THREADS)]

    def worker(t):
        def fn():
            h = streams[t].cuda_stream
            for r in range(REPEATS):
                for j in range(len(CASES)):
                    k = (j + t + r) % len(CASES)   # threads interleave different cases
                    x, wp, wdp, nb, _, _ = prepared[k]
                    status[t].append(_call(CASES[k], x, wp, wdp, outs[t][k], wss[t][k], nb, h))
        return fn

    say("threads", THREADS, "x", REPEATS, "rounds over", len(CASES), "cases")
    _run_threads([worker(t) for t in range(THREADS)])
    torch.cuda.synchronize()
    for t in range(THREADS):
        assert all(s == sw.SWIGLU_OK for s in status[t]), status[t]
        for k, case in enumerate(CASES):
            assert torch.equal(outs[t][k], refs[k]), ("thread", t, "case", case)


def test_threads_noalloc_first_calls_concurrent():
    # a shape whose plan uses no workspace (one kernel, no split): the calls
    # touch no shared memory, so the threads run on their own streams and
    # what they exercise concurrently is the host side, including each
    # device's first-call lookup of the array's address
    torch = torch_mod()
    sw = _sw()
    case = (1, 512, 1024, BF16, False)
    M, d, dff, dt, _ = case
    assert sw.swiglu_workspace_bytes(M, d, dff, dt, 0) == 0
    x, wp, _, nb, shape, odt = _prepare(case, 5200)
    ref = empty(shape, odt)
    sw.check(sw.swiglu_up(x, wp, ref, M, d, dff, dt, None, 0), "reference call")
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(THREADS)]
    outs = [empty(shape, odt) for _ in range(THREADS)]
    status = [[] for _ in range(THREADS)]

    def worker(t):
        def fn():
            h = streams[t].cuda_stream
            for _ in range(REPEATS):
                status[t].append(sw.swiglu_up_noalloc(x, wp, outs[t], M, d, dff, dt, h))
        return fn

    say("noalloc threads", THREADS, "own streams, no workspace")
    _run_threads([worker(t) for t in range(THREADS)])
    torch.cuda.synchronize()
    for t in range(THREADS):
        assert all(s == sw.SWIGLU_OK for s in status[t]), status[t]
        assert torch.equal(outs[t], ref), ("thread", t)


def test_threads_noalloc_serialised_on_one_stream():
    # the documented rule for calls that use the array: one stream, one call
    # at a time (a lock).  Each thread has its own inputs, so a second pass
    # that read another call's partial sums would show in the results.
    import threading as th
    torch = torch_mod()
    sw = _sw()
    M, d, dff, dt = 2, 4096, 2048, BF16
    assert sw.swiglu_workspace_bytes(M, d, dff, dt, 0) > 0   # split K: the array is used
    prepared = [_prepare((M, d, dff, dt, False), 5300 + t) for t in range(THREADS)]
    refs = []
    for x, wp, _, nb, shape, odt in prepared:
        ref = empty(shape, odt)
        sw.check(sw.swiglu_up(x, wp, ref, M, d, dff, dt, bytes_buf(nb), nb), "reference call")
        refs.append(ref)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    h = stream.cuda_stream
    lock = th.Lock()
    outs = [empty(p[4], p[5]) for p in prepared]
    status = [[] for _ in range(THREADS)]

    def worker(t):
        def fn():
            x, wp = prepared[t][0], prepared[t][1]
            for _ in range(REPEATS):
                with lock:
                    status[t].append(sw.swiglu_up_noalloc(x, wp, outs[t], M, d, dff, dt, h))
        return fn

    say("noalloc threads", THREADS, "serialised on one stream")
    _run_threads([worker(t) for t in range(THREADS)])
    torch.cuda.synchronize()
    for t in range(THREADS):
        assert all(s == sw.SWIGLU_OK for s in status[t]), status[t]
        assert torch.equal(outs[t], refs[t]), ("thread", t)


def test_threads_outputs_are_not_trivial():
    # guards the test above against comparing two untouched buffers: the
    # reference of the first case is finite and not all zero
    torch = torch_mod()
    sw = _sw()
    case = CASES[0]
    x, wp, wdp, nb, shape, odt = _prepare(case, 5100)
    out = empty(shape, odt)
    out.fill_(0)
    sw.check(_call(case, x, wp, wdp, out, bytes_buf(nb), nb, None), "call")
    torch.cuda.synchronize()
    vals = wl.bf16_bits_to_f32(out.cpu().numpy().view(np.uint16))
    assert np.isfinite(vals).all() and np.abs(vals).max() > 0
