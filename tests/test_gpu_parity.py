"""GPU parity of the HIP path against the CPU oracle, through the C ABI, at
sizes the oracle finishes quickly that still span several tiles and ragged
tails, on both paths; plus exact closed forms (integer inputs, zero and
one-hot rows), bitwise metamorphic relations, determinism and the packed
layout round trip."""
import numpy as np
import torch  # noqa: F401  (first import on a fresh box is slow; keep it out of test timeouts)
import pytest

import gemv_gate_up_amd as sw
import oracle
import workloads as wl
from swiglu_testlib import (TOL, assert_close, bytes_buf, compare, dev, host, pack, run_mlp,
                            run_up, say, torch_mod)

pytestmark = pytest.mark.gpu

SKINNY, WIDE, AUTO = sw.SWIGLU_PATH_SKINNY, sw.SWIGLU_PATH_WIDE, sw.SWIGLU_PATH_AUTO
PHASED = sw.SWIGLU_PATH_WIDE_PHASED
BF16, F32 = wl.BF16, wl.F32


def _decode(a):
    return a.astype(np.float64) if a.dtype == np.float32 else wl.bf16_bits_to_f32(a).astype(np.float64)


# ---------------------------------------------------------------- packed layout
def unpack_gateup(buf: np.ndarray, d: int, dff: int, dtype: int):
    """Host reading of the packed layout: [pair block][chunk][half][k-group]
    [column][VE values]; returns (Wg, Wu) and the padding."""
    ve = 8 if dtype == BF16 else 4
    kc_len = 4 * ve
    nkc = -(-d // (2 * kc_len)) * 2
    npb = -(-(-(-dff // 16)) // 8) * 8
    arr = buf.view(np.uint16 if dtype == BF16 else np.float32)
    arr = arr.reshape(npb, nkc, 2, 4, 16, ve)
    full = arr.transpose(2, 1, 3, 5, 0, 4).reshape(2, nkc * kc_len, npb * 16)
    return full[0], full[1]


def unpack_down(buf: np.ndarray, d: int, dff: int, dtype: int):
    ve = 8 if dtype == BF16 else 4
    kc_len = 4 * ve
    nkc = -(-dff // (2 * kc_len)) * 2
    npb = -(-(-(-d // 32)) // 8) * 8
    arr = buf.view(np.uint16 if dtype == BF16 else np.float32)
    arr = arr.reshape(npb, nkc, 2, 4, 16, ve)
    return arr.transpose(1, 3, 5, 0, 2, 4).reshape(nkc * kc_len, npb * 32)


@pytest.mark.parametrize("dtype", [BF16, F32])
@pytest.mark.parametrize("d,dff", [(64, 16), (512, 2048), (200, 120), (1000, 1400), (72, 264)])
def test_pack_roundtrip_bitwise(dtype, d, dff):
    say("pack roundtrip", dtype, d, dff)
    inp = wl.random_inputs(3, 1, d, dff, dtype, with_down=True)
    wp, wdp = pack(inp, d, dff, dtype)
    torch_mod().cuda.synchronize()
    raw = wp.cpu().numpy()
    assert raw.size == sw.swiglu_packed_bytes(d, dff, dtype)
    g, u = unpack_gateup(raw, d, dff, dtype)
    assert np.array_equal(g[:d, :dff], inp["wg"]) and np.array_equal(u[:d, :dff], inp["wu"])
    g[:d, :dff] = 0
    u[:d, :dff] = 0
    assert not g.any() and not u.any(), "padding must be zero"
    rawd = wdp.cpu().numpy()
    wd = unpack_down(rawd, d, dff, dtype)
    assert np.array_equal(wd[:dff, :d], inp["wd"])
    wd[:dff, :d] = 0
    assert not wd.any()


# ---------------------------------------------------------------- random parity
# (M, d, dff): tile-spanning shapes with ragged tails in M, d (K) and dff (N).
# Three have at least 512 pair blocks at 17-64 rows, where the skinny path
# takes four pair blocks per workgroup (two, three and four row tiles); the
# last has 1,184 pair blocks at 16 rows, where two per workgroup balance the
# CUs better than four.
BF16_UP_SHAPES = [
    (1, 512, 2048), (3, 264, 200), (16, 1032, 776), (17, 520, 1048), (40, 136, 3000),
    (64, 896, 4864), (65, 256, 264), (100, 328, 1000), (300, 1000, 1400), (513, 64, 512),
    (20, 264, 8200), (40, 520, 8200), (64, 1032, 8200), (16, 264, 18944),
]


@pytest.mark.parametrize("shape", BF16_UP_SHAPES)
@pytest.mark.parametrize("path", [AUTO, SKINNY, WIDE, PHASED])
def test_up_bf16_random(shape, path):
    M, d, dff = shape
    say("up bf16", shape, "path", path)
    inp = wl.random_inputs(M * 7 + d, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    out = host(run_up(dev(inp["x"]), wp, M, d, dff, BF16, path), BF16)
    ref = oracle.swiglu(inp["x"], inp["wg"], inp["wu"])
    assert_close(out, ref, BF16, "up bf16 %s path %d" % (shape, path))


# from three rows on fp32 takes the matrix-unit kernel: 5, 9 and 33 rows
# (one, one and three row tiles), and on larger matrices a partial tile of 12
# rows and 20 rows as one full tile and a partial one; up to two rows, a
# product of fewer pair blocks than half the CUs shares each pair block
# between workgroups (1 x 512 x 2048, 2 x 36 x 20, 2 x 264 x 1000)
F32_SHAPES = [(1, 512, 2048), (2, 36, 20), (5, 100, 60), (9, 260, 132), (33, 64, 2048),
              (12, 520, 8200), (20, 264, 8200), (2, 264, 1000)]


@pytest.mark.parametrize("shape", F32_SHAPES)
def test_up_f32_random(shape):
    M, d, dff = shape
    say("up f32", shape)
    inp = wl.random_inputs(M + d, M, d, dff, F32)
    wp, _ = pack(inp, d, dff, F32)
    out = host(run_up(dev(inp["x"]), wp, M, d, dff, F32), F32)
    ref = oracle.swiglu(inp["x"], inp["wg"], inp["wu"])
    assert_close(out, ref, F32, "up f32 %s" % (shape,))


MLP_SHAPES = [(1, 256, 512, BF16), (7, 136, 392, BF16), (64, 896, 4864, BF16),
              (130, 264, 712, BF16), (4, 100, 60, F32), (12, 64, 520, F32),
              (20, 264, 8200, F32), (1, 200, 1000, F32), (2, 600, 100, F32)]


@pytest.mark.parametrize("shape", MLP_SHAPES)
@pytest.mark.parametrize("path", [AUTO, SKINNY, WIDE, PHASED])
def test_mlp_random(shape, path):
    M, d, dff, dtype = shape
    say("mlp", shape, "path", path)
    inp = wl.random_inputs(M + 3 * d, M, d, dff, dtype, with_down=True)
    wp, wdp = pack(inp, d, dff, dtype)
    if path in (WIDE, PHASED) and dtype == F32:
        # the wide path is bf16 only: the forced call is rejected before any
        # launch and leaves the output as it was
        y = dev(np.full((M, d), 7.0, np.float32))
        ws = bytes_buf(1 << 20)
        rc = sw.mlp_forward_ex(dev(inp["x"]), wp, wdp, y, M, d, dff, dtype, ws, 1 << 20, None, path)
        torch_mod().cuda.synchronize()
        assert rc == sw.SWIGLU_ERR_UNSUPPORTED
        assert np.all(y.cpu().numpy() == 7.0)
        return
    y = host(run_mlp(dev(inp["x"]), wp, wdp, M, d, dff, dtype, path), dtype)
    ref = oracle.mlp(inp["x"], inp["wg"], inp["wu"], inp["wd"])
    assert_close(y, ref, dtype, "mlp %s path %d" % (shape, path))


# ---------------------------------------------------------------- exact closed forms
@pytest.mark.parametrize("dtype,path", [(BF16, SKINNY), (BF16, WIDE), (BF16, PHASED),
                                        (F32, SKINNY)])
def test_integer_inputs_exact_products(dtype, path):
    # |x|, |w| <= 4 and d <= 1000: every product and partial sum is an integer
    # below 2^24, exact in fp32 in any order, so only silu and the final
    # rounding separate the GPU from the oracle.
    M, d, dff = (12, 1000, 520) if path == SKINNY else (80, 1000, 520)
    say("integer exact", dtype, path)
    inp = wl.integer_inputs(5, M, d, dff, dtype)
    wp, _ = pack(inp, d, dff, dtype)
    out = host(run_up(dev(inp["x"]), wp, M, d, dff, dtype, path), dtype)
    ref = oracle.swiglu(inp["x"], inp["wg"], inp["wu"])
    rel = 2.0 ** -8 + 1e-5 if dtype == BF16 else 1e-5
    bound = rel * np.abs(ref) + 1e-30
    assert np.all(np.abs(out - ref) <= bound), compare(out, ref, rel)


@pytest.mark.parametrize("path", [SKINNY, WIDE, PHASED])
def test_zero_input_gives_exact_zero(path):
    M, d, dff = 70, 256, 384
    inp = wl.random_inputs(9, M, d, dff, BF16, with_down=True)
    wp, wdp = pack(inp, d, dff, BF16)
    x0 = dev(np.zeros_like(inp["x"]))
    assert not host(run_up(x0, wp, M, d, dff, BF16, path), BF16).any()
    assert not host(run_mlp(x0, wp, wdp, M, d, dff, BF16, path), BF16).any()


@pytest.mark.parametrize("path", [SKINNY, WIDE, PHASED])
def test_one_hot_rows_select_weight_rows(path):
    M, d, dff = 72, 320, 264
    ks = [(37 * m) % d for m in range(M)]
    x = wl.one_hot_rows(M, d, ks, BF16)
    w = wl.random_inputs(13, 1, d, dff, BF16)
    wp, _ = pack(w, d, dff, BF16)
    out = host(run_up(dev(x), wp, M, d, dff, BF16, path), BF16)
    ref = oracle.swiglu(x, w["wg"], w["wu"])
    # g and u are exactly rows of Wg and Wu: only silu and the rounding remain
    assert np.all(np.abs(out - ref) <= (2.0 ** -8 + 1e-5) * np.abs(ref) + 1e-30)


# ---------------------------------------------------------------- metamorphic (bitwise)
@pytest.mark.parametrize("path", [SKINNY, WIDE, PHASED])
def test_determinism_bitwise(path):
    M, d, dff = (16, 2048, 3072) if path == SKINNY else (300, 1024, 1536)
    inp = wl.random_inputs(17, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    x = dev(inp["x"])
    a = run_up(x, wp, M, d, dff, BF16, path).cpu().numpy()
    b = run_up(x, wp, M, d, dff, BF16, path).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("path", [SKINNY, WIDE, PHASED])
def test_linearity_in_up_weight_bitwise(path):
    # out(x, Wg, 2 Wu) = 2 out(x, Wg, Wu): power-of-two scaling is exact
    M, d, dff = (8, 512, 640) if path == SKINNY else (128, 512, 640)
    inp = wl.random_inputs(19, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    inp2 = dict(inp)
    inp2["wu"] = wl.f32_to_bf16_bits(2.0 * wl.bf16_bits_to_f32(inp["wu"]))
    wp2, _ = pack(inp2, d, dff, BF16)
    x = dev(inp["x"])
    o1 = host(run_up(x, wp, M, d, dff, BF16, path), BF16)
    o2 = host(run_up(x, wp2, M, d, dff, BF16, path), BF16)
    assert np.array_equal(o2, 2.0 * o1)


@pytest.mark.parametrize("path", [SKINNY, WIDE, PHASED])
def test_joint_column_permutation_bitwise(path):
    M, d, dff = (4, 256, 512) if path == SKINNY else (96, 256, 512)
    inp = wl.random_inputs(23, M, d, dff, BF16)
    perm = np.random.default_rng(0).permutation(dff)
    inp2 = dict(inp, wg=np.ascontiguousarray(inp["wg"][:, perm]),
                wu=np.ascontiguousarray(inp["wu"][:, perm]))
    wp, _ = pack(inp, d, dff, BF16)
    wp2, _ = pack(inp2, d, dff, BF16)
    x = dev(inp["x"])
    o1 = run_up(x, wp, M, d, dff, BF16, path).cpu().numpy()
    o2 = run_up(x, wp2, M, d, dff, BF16, path).cpu().numpy()
    assert np.array_equal(o2, o1[:, perm])


def test_gate_up_swap_changes_result():
    M, d, dff = 4, 128, 256
    inp = wl.random_inputs(29, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    wps, _ = pack(dict(inp, wg=inp["wu"], wu=inp["wg"]), d, dff, BF16)
    x = dev(inp["x"])
    o1 = host(run_up(x, wp, M, d, dff, BF16), BF16)
    o2 = host(run_up(x, wps, M, d, dff, BF16), BF16)
    assert not np.allclose(o1, o2, atol=1e-2)
    assert_close(o1, oracle.swiglu(inp["x"], inp["wg"], inp["wu"]), BF16)


def test_rows_are_independent_on_the_skinny_path():
    # Each row's sums run in the same order whatever M <= 64 is, so a row of
    # a 16-row call equals the one-row call on that row, bit for bit.
    M, d, dff = 16, 1024, 1280
    inp = wl.random_inputs(31, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    full = run_up(dev(inp["x"]), wp, M, d, dff, BF16, SKINNY).cpu().numpy()
    for m in (0, 5, 15):
        one = run_up(dev(inp["x"][m:m + 1]), wp, 1, d, dff, BF16, SKINNY).cpu().numpy()
        assert np.array_equal(one[0], full[m]), m


def test_paths_agree_where_both_apply():
    M, d, dff = 96, 768, 1024
    inp = wl.random_inputs(37, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    x = dev(inp["x"])
    a = host(run_up(x, wp, M, d, dff, BF16, SKINNY), BF16)
    b = host(run_up(x, wp, M, d, dff, BF16, WIDE), BF16)
    ref = oracle.swiglu(inp["x"], inp["wg"], inp["wu"])
    assert_close(a, ref, BF16)
    assert_close(b, ref, BF16)
    # two correct fp32-accumulated orders differ by at most a couple of bf16 ulps
    assert np.all(np.abs(a - b) <= 2 * 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-3)


# The one-pass schedule picks its tile from the grid: 128 x 128 up to 128 rows
# and 256 x 128 above while a grid of 256 x 256 tiles would have at most 128
# of them, 256 x 256 otherwise.  (128, 256, 1024) and (129, 256, 1024) sit on
# either side of the row boundary, (256, 64, 16384) and (256, 64, 16512) on
# either side of the tile-count boundary (128 and 129 tiles), (1024, 256,
# 4224) has 132 tiles of 256 x 256.
@pytest.mark.parametrize("shape", [(96, 768, 1024), (300, 1000, 1400), (257, 520, 2056),
                                   (1024, 4096, 1536), (128, 256, 1024), (129, 256, 1024),
                                   (256, 64, 16384), (256, 64, 16512), (1024, 256, 4224)])
def test_two_pass_schedule_is_bitwise_the_one_pass_result(shape):
    # Both schedules sum every accumulator over the same MFMAs in the same
    # K order and apply silu(gate) * up in fp32, so they agree bit for bit.
    M, d, dff = shape
    say("phased vs wide", shape)
    inp = wl.random_inputs(43 + M, M, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    x = dev(inp["x"])
    a = run_up(x, wp, M, d, dff, BF16, WIDE).cpu().numpy()
    b = run_up(x, wp, M, d, dff, BF16, PHASED).cpu().numpy()
    assert np.array_equal(a, b)


def test_empty_batch_is_a_noop():
    d, dff = 64, 64
    inp = wl.random_inputs(41, 1, d, dff, BF16)
    wp, _ = pack(inp, d, dff, BF16)
    out = dev(np.full((1, dff), 0x7FC0, dtype=np.uint16))
    assert sw.swiglu_up(dev(inp["x"]), wp, out, 0, d, dff, BF16) == sw.SWIGLU_OK
    torch_mod().cuda.synchronize()
    assert np.all(out.cpu().numpy().view(np.uint16) == 0x7FC0)
