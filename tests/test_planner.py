"""The split-K planner of the few-rows path (plan_skinny in csrc/skinny.hip),
restated in plain Python and checked through the size queries of the C ABI
(no GPU is used).  On the forced few-rows path the workspace of swiglu_up is
the gate/up product's split-K partials, and that of mlp_forward is h plus the
larger of the two products' partials (its gate/up product writes h at the
padded width of 128-column multiples); each product's partials are
slices x M x (packed columns) x 4 bytes when K is split.  The rule:

* A product has grid_pb output blocks (16 gate/up columns, or 32 down
  columns, each) and row groups of 16 x min(4, ceil(M / 16)) rows (fp32 at
  one and two rows: groups of one and two rows).
* K is split in two, four, ... while the blocks times the slices are below
  the target (one workgroup per CU, 256, for a gate/up product whose row
  group holds more than 16 rows; two per CU otherwise), each slice keeps at
  least 16 K chunks of the packed weight, and fewer than 64 slices.
* No split at all when the packed weight holds under 128 KiB per output
  block, where the second pass would cost more than it saves.
* The slice count is then rounded to the chunks: ceil(nkc / ceil(nkc / S)).
"""
import itertools

import pytest

import gemv_gate_up_amd as sw
import workloads as wl

BF16, F32, W8, W4 = wl.BF16, wl.F32, wl.FP8W, wl.MXFP4W
SKINNY = sw.SWIGLU_PATH_SKINNY
CUS = 256


def _cdiv(a, b):
    return -(-a // b)


def _geom(K, N, cols, dt):
    """Chunks along K, padded output blocks and packed bytes of one weight."""
    chunk = {F32: 16, BF16: 32, W8: 64, W4: 128}[dt]
    align = chunk if dt in (W8, W4) else 2 * chunk
    nkc = _cdiv(K, align) * align // chunk
    npb = _cdiv(_cdiv(N, cols), 8) * 8
    nbytes = npb * nkc * 2 * 1024
    if dt == W8:
        nbytes += npb * 32 * 4
    if dt == W4:
        nbytes += npb * nkc * 2 * 64
    return nkc, npb, nbytes


def _slices(M, K, N, cols, dt, gate_up):
    nkc, npb, nbytes = _geom(K, N, cols, dt)
    grid_pb = _cdiv(N, cols)
    if dt == F32 and M < 3:
        row_tile = 2 if M >= 2 else 1
    else:
        row_tile = 16 * min(4, max(1, _cdiv(M, 16)))
    base = grid_pb * _cdiv(M, row_tile)
    target = CUS if (gate_up and row_tile > 16) else 2 * CUS
    S = 1
    if nbytes >= 128 * 1024 * grid_pb:
        while base * S < target and nkc // (2 * S) >= 16 and S < 64:
            S *= 2
    S = _cdiv(nkc, _cdiv(nkc, S))
    return S, npb


def _partials(M, K, N, cols, dt, gate_up):
    S, npb = _slices(M, K, N, cols, dt, gate_up)
    return S * M * npb * 32 * 4 if S > 1 else 0


def _al(n):
    return _cdiv(n, 256) * 256


def _expected(M, d, dff, dt, with_down):
    pu = _partials(M, d, dff, 16, dt, True)
    if not with_down:
        return _al(pu)
    # the MLP's gate/up product writes h at its padded width: its blocks
    # include the padding
    padded = _cdiv(_cdiv(dff, 16), 8) * 8 * 16
    pu = _partials(M, d, padded, 16, dt, True)
    pd = _partials(M, dff, d, 32, dt, False)
    h = M * padded * (4 if dt == F32 else 2)
    return _al(h) + _al(max(pu, pd))


ROWS = [1, 2, 3, 5, 8, 16, 17, 33, 64, 65, 130]
DIMS = [64, 520, 1000, 4096]
FFS = [40, 1048, 4864, 14336]


@pytest.mark.parametrize("dt", [BF16, F32, W8, W4])
def test_few_rows_workspace_follows_the_split_rule(dt):
    bad = []
    for M, d, dff, down in itertools.product(ROWS, DIMS, FFS, (0, 1)):
        got = sw.swiglu_workspace_bytes_ex(M, d, dff, dt, down, SKINNY)
        want = _expected(M, d, dff, dt, down)
        if got != want:
            bad.append(((M, d, dff, down), got, want))
    assert not bad, bad[:10]


def test_the_rule_splits_where_blocks_are_few():
    # the restated rule itself on the shapes the comments of plan_skinny name:
    # the 8B decode fills the GPU unsplit, a long K over few blocks splits,
    # the tiny fp32 decode streams too little per block to split, and the
    # 0.5B-class MLP's down product at 64 rows splits eight ways
    assert _slices(1, 4096, 14336, 16, BF16, True)[0] == 1
    assert _slices(1, 4096, 512, 16, F32, True)[0] == 16
    assert _slices(1, 512, 2048, 16, F32, True)[0] == 1
    assert _slices(64, 4864, 896, 32, BF16, False)[0] == 8
    assert _slices(64, 896, 4864, 16, BF16, True)[0] == 1


# ---------------------------------------------------------------- dispatcher
# The automatic path of a gate/up product (swiglu_select_path): bf16 above
# 64 rows takes the wide MFMA kernel when its grid keeps the chip busy, and
# every other product the few-rows kernels.  The wide grid counts 256 x 256
# tiles (8 pair blocks of 16 gate + 16 up columns across); a grid of at most
# 128 of them runs as narrower tiles instead, 128 x 128 up to 128 rows and
# 256 x 128 above, and the dispatcher counts those.  Wide when that count is
# at least 128, or at least 48 from 256 rows on.

def _wide_tiles(M, dff):
    pbs = _cdiv(dff, 16)
    full = _cdiv(M, 256) * _cdiv(pbs, 8)
    if full > CUS // 2:
        return full
    return _cdiv(M, 128 if M <= 128 else 256) * _cdiv(pbs, 4)


def _auto_path(M, d, dff, dt):
    if dt == BF16 and M > 64:
        t = _wide_tiles(M, dff)
        if t >= CUS // 2 or (M >= 256 and t >= 48):
            return sw.SWIGLU_PATH_WIDE
    return SKINNY


@pytest.mark.parametrize("dt", [BF16, F32, W8, W4])
def test_automatic_path_follows_the_grid_rule(dt):
    bad = []
    for M, d, dff in itertools.product(
            [1, 16, 64, 65, 96, 128, 129, 192, 255, 256, 300, 512, 1024, 4096],
            [896, 1536, 4096, 8192], [896, 3696, 4864, 8960, 14336, 29568]):
        got = sw.swiglu_select_path(M, d, dff, dt)
        if got != _auto_path(M, d, dff, dt):
            bad.append(((M, d, dff), got))
    assert not bad, bad[:10]


def test_the_grid_rule_on_named_shapes():
    # the 8B prefill and the 72B MLP's products are wide; the 0.5B-class
    # gate/up product (76 narrow tiles from 129 to 256 rows) stays on the
    # few-rows kernels below 256 rows and goes wide at 256; the 8B shape
    # takes the wide kernel from 65 rows (224 narrow tiles)
    assert _auto_path(4096, 4096, 14336, BF16) == sw.SWIGLU_PATH_WIDE
    assert _auto_path(2048, 8192, 29568, BF16) == sw.SWIGLU_PATH_WIDE
    assert _wide_tiles(255, 4864) == _wide_tiles(256, 4864) == 76
    assert _auto_path(255, 896, 4864, BF16) == SKINNY
    assert _auto_path(256, 896, 4864, BF16) == sw.SWIGLU_PATH_WIDE
    assert _auto_path(65, 4096, 14336, BF16) == sw.SWIGLU_PATH_WIDE
    assert _wide_tiles(65, 14336) == 224
