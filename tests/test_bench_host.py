"""Host-side logic of bench.py that needs no GPU: the run order and the power
sampler's parsing of `amd-smi metric -p -c` and its sample window."""
import subprocess

import bench

# The shape of `amd-smi metric -p -c` on one MI355X (two of eight graphics
# partitions shown; the values are illustrative).
SMI_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1393 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1889 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1968 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 2000 MHz
"""


def test_run_order_keeps_default_order_then_extras():
    names = bench.CONFIGS + bench.QUANT_CONFIGS
    assert bench.run_order([]) == names
    picked = [names[3], names[1]]
    assert bench.run_order(picked) == [names[1], names[3]]
    assert bench.run_order(["prefill8b_m256", names[0]]) == [names[0], "prefill8b_m256"]


def test_power_sampler_parses_socket_power_and_graphics_clocks(monkeypatch):
    class Done:
        stdout = SMI_TEXT

    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Done())
    p = bench.PowerSampler()
    watts, clks = p._read()
    assert watts == 1393.0
    assert clks == [1889.0, 1968.0]   # graphics partitions only, not the memory clock


def test_power_sampler_unparsable_output_gives_no_sample(monkeypatch):
    class Done:
        stdout = "ERROR: no devices"

    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Done())
    assert bench.PowerSampler()._read() is None


def test_power_sampler_window_drops_samples_before_skip():
    p = bench.PowerSampler(skip_s=1.0)
    p.t0, p.t1 = 100.0, 105.0
    p.samples = [(100.5, 900.0, [1000.0]), (101.5, 1390.0, [1900.0, 1950.0]),
                 (104.0, 1396.0, [1880.0, 1960.0]), (105.5, 500.0, [100.0])]
    s = p.summary()
    assert s["samples"] == 2
    assert s["socket_w_mean"] == 1393.0
    assert s["socket_w_max"] == 1396.0
    assert s["gfx_mhz_min"] == 1880.0 and s["gfx_mhz_max"] == 1960.0
    assert s["gfx_mhz_mean"] == round((1925.0 + 1920.0) / 2, 1)


def test_power_window_fraction_at_the_sampled_clock(monkeypatch):
    # the extra steps run through measure(); here they only feed the sampler
    class FakeSampler:
        def __init__(self, skip_s=0.5):
            self.skip_s = skip_s

        def summary(self):
            return {"samples": 3, "gfx_mhz_mean": 1800.0}

    monkeypatch.setattr(bench, "PowerSampler", FakeSampler)
    seen = {}

    def fake_measure(w, inputs, steps, warmup, copies, check=True, window=None, markers=True,
                     read_ceilings=True):
        seen.update(steps=steps, check=check, window=window, markers=markers,
                    read_ceilings=read_ceilings)
        return {}

    monkeypatch.setattr(bench, "measure", fake_measure)
    rec = {"roofline": {"event_ms_per_step": 0.5, "achieved": 1320.0}}
    out = bench.power_window(bench.wl.WORKLOADS["prefill8b_m4096"], None, rec, 2.5, 1)
    assert seen["steps"] == 5000 and seen["check"] is False and seen["markers"] is False
    assert seen["read_ceilings"] is False
    assert isinstance(seen["window"], FakeSampler) and seen["window"].skip_s == 1.0
    at_clock = bench.BF16_PEAK_TFLOPS * 1800.0 / 2400.0
    assert out["peak_at_clock_tflops"] == round(at_clock, 1)
    assert out["frac_at_clock"] == round(1320.0 / at_clock, 4)
    assert out["steps"] == 5000


def test_max_ulps_at_bf16_and_fp32_precision():
    import numpy as np
    ref = np.array([1.0, -3.0, 0.0])
    err = np.array([2.0 ** -8, 2.0 ** -7, 5.0])   # 0.5 ulp of 1 (2^-7), 0.5 ulp of 3 (2^-6); zero skipped
    assert bench.max_ulps(err, ref, 7) == 0.5
    assert bench.max_ulps(np.array([2.0 ** -23]), np.array([1.0]), 23) == 1.0
    assert bench.max_ulps(np.array([1.0]), np.array([0.0]), 7) == 0.0


def _decoded(inp):
    import oracle
    return {k: oracle.to_double(v) for k, v in inp.items()}


def test_dot_scale_of_swiglu_outputs():
    # against numpy on the decoded values: |d h/d g| sum|x||wg| + |d h/d u| sum|x||wu|
    import numpy as np
    w = bench.wl.Workload(0, "t", 3, 16, 24, bench.wl.BF16, False, 3)
    inp = bench.wl.random_inputs(77, 3, 16, 24, bench.wl.BF16)
    got = bench.dot_scale(w, inp["x"], {"wg": inp["wg"], "wu": inp["wu"]}, None)
    f = _decoded(inp)
    g, u = f["x"] @ f["wg"], f["x"] @ f["wu"]
    sg, su = np.abs(f["x"]) @ np.abs(f["wg"]), np.abs(f["x"]) @ np.abs(f["wu"])
    sig = 1.0 / (1.0 + np.exp(-g))
    want = np.abs(u * sig * (1 + g * (1 - sig))) * sg + np.abs(g * sig) * su
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=0)   # float32 arithmetic


def test_dot_scale_of_mlp_outputs():
    import numpy as np
    import oracle
    w = bench.wl.Workload(0, "t", 2, 16, 24, bench.wl.BF16, True, 2)
    inp = bench.wl.random_inputs(78, 2, 16, 24, bench.wl.BF16, with_down=True)
    wts = {k: inp[k] for k in ("wg", "wu", "wd")}
    got = bench.dot_scale(w, inp["x"], wts, [1])
    f = _decoded(inp)
    h = oracle.swiglu(inp["x"], inp["wg"], inp["wu"])
    want = np.abs(h[1:2]) @ np.abs(f["wd"])
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=0)


def test_accuracy_record_reports_the_new_diagnostics():
    import numpy as np
    ref = np.array([[1.0, 2.0]])
    got = ref + np.array([[2.0 ** -9, 0.0]])
    rec = bench.accuracy(got, ref, 2e-2, "test", np.array([[0.5, 0.0]]), 7)
    assert rec["ok"] and rec["max_ulps"] == 0.25
    assert rec["max_err_over_dot_scale"] == 2.0 ** -9 / 0.5


def test_as_f32_decodes_each_storage():
    import numpy as np
    import oracle
    w = bench.wl.to_storage(bench.wl.normal(5, (8, 16), 0.5), bench.wl.BF16)
    np.testing.assert_array_equal(bench._as_f32(w).astype(np.float64), oracle.to_double(w))
    codes, scales = oracle.quantize_e4m3(w)
    np.testing.assert_allclose(bench._as_f32((codes, scales)),
                               oracle.dequantize_e4m3(codes, scales), rtol=1e-7, atol=0)
