"""Checks of the seeded input generator (host only)."""
import numpy as np

import workloads as wl


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    cases = {
        1.0: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,          # halfway, ties to even (down)
        1.0 + 3 * 2.0 ** -8: 0x3F82,      # halfway, ties to even (up)
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,   # just above halfway
        -2.0: 0xC000,
    }
    for v, bits in cases.items():
        assert int(wl.f32_to_bf16_bits(np.array([v], dtype=np.float32))[0]) == bits, v
    assert one == wl.bf16_bits_to_f32(np.array([0x3F80], dtype=np.uint16))[0]


def test_bf16_roundtrip_is_identity_on_bf16_values():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(bits)), bits)


def test_bf16_rounding_error_bound():
    a = wl.normal(5, (100000,), 1.0)
    r = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(a)).astype(np.float64)
    rel = np.abs(r - a) / np.abs(a)
    assert rel.max() <= 2.0 ** -8


def test_seeds_reproducible_and_distinct():
    w = wl.WORKLOADS["tiny_decode_f32"]
    a = wl.make_inputs(w)
    b = wl.make_inputs(w)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["wg"], a["wu"])


def test_distributions_match_workload_recipe():
    w = wl.WORKLOADS["mlp05b_m64"]
    inp = wl.make_inputs(w)
    assert inp["x"].shape == (64, 896) and inp["x"].dtype == np.uint16
    assert inp["wg"].shape == (896, 4864) and inp["wd"].shape == (4864, 896)
    x = wl.bf16_bits_to_f32(inp["x"])
    wg = wl.bf16_bits_to_f32(inp["wg"])
    wd = wl.bf16_bits_to_f32(inp["wd"])
    assert abs(x.std() - 1.0) < 0.02
    assert abs(wg.std() * np.sqrt(896) - 1.0) < 0.01
    assert abs(wd.std() * np.sqrt(4864) - 1.0) < 0.01


def test_smaller_m_takes_leading_rows():
    a = wl.make_inputs(wl.WORKLOADS["decode8b_m4"])["x"]
    b = wl.make_inputs(wl.WORKLOADS["decode8b_m16"])["x"]
    assert np.array_equal(a, b[:4])


def test_algorithmic_counts():
    w = wl.WORKLOADS["decode8b_m1"]
    assert 2 * w.d * w.dff * 2 == 234881024
    assert w.algorithmic_bytes() == 234917888
    assert wl.WORKLOADS["prefill8b_m4096"].algorithmic_flops() == 4 * 4096 * 4096 * 14336
    assert wl.WORKLOADS["mlp72b_m16"].algorithmic_bytes() == 1453850624
