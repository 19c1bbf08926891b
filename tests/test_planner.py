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
