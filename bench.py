#!/usr/bin/env python3
"""Benchmark of the fused SwiGLU MLP hot path on one MI355X.

One step = one call of the hot path (swiglu_up / mlp_forward through the C
ABI) on resident inputs.  The headline line is the 8B-class decode step
(M = 1, d = 4096, d_ff = 14336, bf16) in HBM GB/s of algorithmic traffic
(both weight matrices once, x once, the output once); the same JSON line also
carries the 8B-class prefill step (M = 4096) in bf16 TFLOP/s.

Weights are rotated through a ring of copies (>= 1 GB in total) so that the
256 MB Infinity Cache cannot serve a repeated call: every timed call streams
its weights from HBM.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
F32_VALU_PEAK_TFLOPS = 157.3
METRIC = "fused SwiGLU MLP: HBM GB/s at M=1 decode; bf16 TFLOP/s at M=4096 prefill"
# sources each kernel's recorded counters depend on
COMMON_SOURCES = ["geometry.h", "device_common.h", "launch.h", "api.hip"]
KERNEL_SOURCES = {
    "skinny_bf16_kernel": COMMON_SOURCES + ["skinny.hip"],
    "skinny_f32_kernel": COMMON_SOURCES + ["skinny.hip"],
    "wide_bf16_kernel": COMMON_SOURCES + ["wide.hip", "wide_kernel.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "gemv_gate_up_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != kernel or rec.get("src_sha") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


class Runner:
    """Device buffers and the C-ABI call for one workload."""

    def __init__(self, w: wl.Workload, copies: int, path: int = 0, graph: bool = False,
                 block: bool = False):
        import torch
        import gemv_gate_up_amd as sw
        self.torch, self.sw, self.w = torch, sw, w
        t0 = time.time()
        self.inp = wl.make_inputs(w, M=w.M)
        log("inputs for %s generated in %.1fs" % (w.name, time.time() - t0))
        tdt = torch.float32 if w.dtype == wl.F32 else torch.int16

        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to("cuda")

        self.x = dev(self.inp["x"])
        wp = torch.empty(sw.swiglu_packed_bytes(w.d, w.dff, w.dtype), dtype=torch.uint8,
                         device="cuda")
        sw.check(sw.swiglu_pack_weights(dev(self.inp["wg"]), dev(self.inp["wu"]), wp, w.d, w.dff,
                                        w.dtype), "pack")
        self.wps = [wp] + [wp.clone() for _ in range(copies - 1)]
        self.wdps = [None] * copies
        if w.with_down:
            wdp = torch.empty(sw.swiglu_down_packed_bytes(w.d, w.dff, w.dtype), dtype=torch.uint8,
                              device="cuda")
            sw.check(sw.swiglu_pack_down(dev(self.inp["wd"]), wdp, w.d, w.dff, w.dtype), "pack")
            self.wdps = [wdp] + [wdp.clone() for _ in range(copies - 1)]
        ncols = w.d if w.with_down else w.dff
        self.out = torch.empty((w.M, ncols), dtype=tdt, device="cuda")
        self.req_path = path
        self.block = block
        if block:
            # the MLP half of a layer: x doubles as the residual stream r;
            # gain and bias drawn like the activations (seeded)
            assert w.with_down, "the block needs the down projection"
            self.gamma = dev(wl.to_storage(1.0 + 0.1 * wl.normal(90, (w.d,), 1.0), w.dtype))
            self.bias = dev(wl.to_storage(wl.normal(91, (w.d,), 0.1), w.dtype))
            self.ws_bytes = sw.mlp_block_workspace_bytes_ex(w.M, w.d, w.dff, w.dtype, path)
        else:
            self.ws_bytes = sw.swiglu_workspace_bytes_ex(w.M, w.d, w.dff, w.dtype,
                                                         int(w.with_down), path)
        if self.ws_bytes < 0:
            raise RuntimeError("path %d: %s" % (path, sw.swiglu_status_string(self.ws_bytes)))
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream()
        self.sh = self.stream.cuda_stream
        self.copies = copies
        self.path = path or sw.swiglu_select_path(w.M, w.d, w.dff, w.dtype)
        # raw pointers once, so a step is a single foreign call
        self.args = [(self.x.data_ptr(), self.wps[i].data_ptr(),
                      self.wdps[i].data_ptr() if self.wdps[i] is not None else None)
                     for i in range(copies)]
        # with graph=True, one recorded call per weight copy; a step replays one
        self.graphs = []
        for i in range(copies if graph else 0):
            xp, wpp, wdpp = self.args[i]
            if w.with_down:
                rc, g = sw.mlp_forward_graph_create(xp, wpp, wdpp, self.out, w.M, w.d, w.dff,
                                                    w.dtype, self.ws, self.ws_bytes, path)
            else:
                rc, g = sw.swiglu_up_graph_create(xp, wpp, self.out, w.M, w.d, w.dff, w.dtype,
                                                  self.ws, self.ws_bytes, path)
            sw.check(rc, "graph create")
            self.graphs.append(g)

    def close(self) -> None:
        for g in self.graphs:
            self.sw.swiglu_graph_destroy(g)
        self.graphs = []

    def step(self, i: int) -> None:
        w, sw = self.w, self.sw
        xp, wpp, wdpp = self.args[i % self.copies]
        if self.block:
            rc = sw._lib.mlp_block_forward_ex(xp, self.gamma.data_ptr(), 1e-6, wpp, wdpp,
                                              self.bias.data_ptr(), self.out.data_ptr(), w.M, w.d,
                                              w.dff, w.dtype, self.ws.data_ptr(), self.ws_bytes,
                                              self.sh, self.req_path)
        elif self.graphs:
            rc = sw._lib.swiglu_graph_launch(self.graphs[i % self.copies], self.sh)
        elif self.req_path and w.with_down:
            rc = sw._lib.mlp_forward_ex(xp, wpp, wdpp, self.out.data_ptr(), w.M, w.d, w.dff,
                                        w.dtype, self.ws.data_ptr(), self.ws_bytes, self.sh,
                                        self.req_path)
        elif self.req_path:
            rc = sw._lib.swiglu_up_ex(xp, wpp, self.out.data_ptr(), w.M, w.d, w.dff, w.dtype,
                                      self.ws.data_ptr(), self.ws_bytes, self.sh, self.req_path)
        elif w.with_down:
            rc = sw._lib.mlp_forward(xp, wpp, wdpp, self.out.data_ptr(), w.M, w.d, w.dff, w.dtype,
                                     self.ws.data_ptr(), self.ws_bytes, self.sh)
        else:
            rc = sw._lib.swiglu_up(xp, wpp, self.out.data_ptr(), w.M, w.d, w.dff, w.dtype,
                                   self.ws.data_ptr(), self.ws_bytes, self.sh)
        if rc != 0:
            raise RuntimeError("step failed: %s" % sw.swiglu_status_string(rc))

    def time(self, steps: int, warmup: int) -> dict:
        """K back-to-back steps between two synchronisations: the host clock
        gives the step rate, and a pair of HIP events recorded on the launch
        stream around the same K launches gives the device time per launch."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(self.stream)
        for i in range(steps):
            self.step(warmup + i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return {"wall_ms_per_step": (t1 - t0) * 1e3 / steps,
                "event_ms_per_launch": e0.elapsed_time(e1) / steps}


PATHS = {"auto": 0, "skinny": 1, "wide": 2, "phased": 3}
PATH_NAMES = {1: "skinny", 2: "wide", 3: "wide-phased"}


def dominant_kernel(w: wl.Workload, path: int) -> str:
    if path in (2, 3):
        return "wide_bf16_kernel"
    return "skinny_f32_kernel" if w.dtype == wl.F32 else "skinny_bf16_kernel"


def block_bytes(w: wl.Workload) -> int:
    """Algorithmic bytes of the MLP block: the MLP's, plus gamma and bias
    (r is the MLP's x, out its y)."""
    return w.algorithmic_bytes() + 2 * w.d * w.elem_bytes


def measure(w: wl.Workload, steps: int, warmup: int, copies: int, path: int = 0,
            graph: bool = False, block: bool = False) -> dict:
    r = Runner(w, copies, path, graph, block)
    t = r.time(steps, warmup)
    kern = dominant_kernel(w, r.path)
    per_launch_ms = t["event_ms_per_launch"]
    single_kernel = (not w.with_down) and (
        r.path in (2, 3) or r.sw.swiglu_workspace_bytes(w.M, w.d, w.dff, w.dtype, 0) == 0)
    res = {"runner": r, "timing": t, "kernel": kern, "path": r.path,
           "single_kernel_step": single_kernel}
    bytes_alg = block_bytes(w) if block else w.algorithmic_bytes()
    flops_alg = w.algorithmic_flops()
    hbm_bound = flops_alg / bytes_alg < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if hbm_bound:
        achieved = bytes_alg / (per_launch_ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = flops_alg / (per_launch_ms * 1e-3) / 1e12
        res["roofline"] = {"bound": "mfma", "achieved": round(achieved, 1),
                           "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    # recorded counters are for the dispatcher's own path
    res["roofline"]["traffic"] = (traffic_from_profile(w.name, kern)
                                  if not (path or graph or block) else None)
    res["roofline"]["kernel"] = kern
    res["roofline"]["kernel_ms"] = round(per_launch_ms, 5)
    if r.path in (2, 3) and not (w.with_down or block or graph):
        # with the reported workspace the many-rows step packs x first; the
        # events span both launches
        res["roofline"]["step_kernels"] = ["pack_act_kernel", kern]
    return res


def cpu_baseline(w: wl.Workload, inp: dict, budget_s: float) -> dict:
    """The oracle, as it stands, on the host cores: full workload calls
    repeated for about budget_s seconds (at least one)."""
    import oracle
    threads = oracle.available_cores()
    x = inp["x"][:w.M]
    if w.dtype == wl.FP8W:   # quantised once, outside the timing
        q = {k: oracle.quantize_e4m3(inp[k]) for k in ("wg", "wu", "wd") if k in inp}
    if w.dtype == wl.MXFP4W:
        q = {k: oracle.dequantize_mxfp4(*oracle.quantize_mxfp4(inp[k]))
             for k in ("wg", "wu", "wd") if k in inp}
        x = oracle.to_double(x)
    reps, t0 = 0, time.perf_counter()
    while True:
        if w.dtype == wl.MXFP4W and w.with_down:
            oracle.mlp(x, q["wg"], q["wu"], q["wd"], nthreads=threads)
        elif w.dtype == wl.MXFP4W:
            oracle.swiglu(x, q["wg"], q["wu"], nthreads=threads)
        elif w.dtype == wl.FP8W and w.with_down:
            oracle.mlp_fp8w(x, *q["wg"], *q["wu"], *q["wd"], nthreads=threads)
        elif w.dtype == wl.FP8W:
            oracle.swiglu_fp8w(x, *q["wg"], *q["wu"], nthreads=threads)
        elif w.with_down:
            oracle.mlp(x, inp["wg"], inp["wu"], inp["wd"], nthreads=threads)
        else:
            oracle.swiglu(x, inp["wg"], inp["wu"], nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per_call = el / reps
    return {"value": round(w.algorithmic_bytes() / per_call / 1e9, 3), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": "%d full %s call(s) (M=%d, d=%d, dff=%d) in %.1f s wall, fp64" % (
                reps, w.name, w.M, w.d, w.dff, el),
            "ms_per_call": round(per_call * 1e3, 2)}


def probe() -> int:
    """Kernels for hardware-counter runs: a plain copy of known size (reads
    and writes exactly 1 GiB) to calibrate FETCH_SIZE / WRITE_SIZE, then the
    decode (bf16, FP8 and MXFP4 weights) and prefill steps as the bench runs them."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    for name, steps in (("decode8b_m1", 5), ("decode8b_m1_fp8w", 5), ("decode8b_m1_mxfp4w", 5),
                        ("prefill8b_m4096", 3)):
        w = wl.WORKLOADS[name]
        r = Runner(w, 5 if w.M == 1 else 1)
        for i in range(steps):
            r.step(i)
        torch.cuda.synchronize()
        del r
        torch.cuda.empty_cache()
    log("probe done")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode8b_m1", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=40,
                    help="untimed prefill steps first: the clock needs ~30 ms of matrix work to settle")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the FP8- and MXFP4-weight decode lines")
    ap.add_argument("--block", action="store_true",
                    help="time the MLP block (RMSNorm, MLP, bias and residual) on a workload "
                         "with the down projection")
    ap.add_argument("--graph", action="store_true",
                    help="replay recorded calls (HIP graphs) instead of direct calls")
    ap.add_argument("--path", default="auto", choices=sorted(PATHS),
                    help="force a kernel path for the main workload (default: the dispatcher's)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--probe", action="store_true",
                    help="counter-collection run: a 1 GiB device copy (calibration), then a few "
                         "steps of the decode and prefill workloads; prints no timing")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(one GPU's share of a sharded MLP is the same kernel at a smaller d_ff).",
              file=sys.stderr)
        return 2

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.probe:
        return probe()
    w = wl.WORKLOADS[args.workload]
    one_copy = int(2 * w.d * w.dff * w.weight_bytes)
    copies = max(1, -(-(1 << 30) // one_copy)) if one_copy < (1 << 30) else 1
    log("workload %s: %s, %d weight copies" % (w.name, w, copies))
    m = measure(w, args.steps, args.warmup, copies, PATHS[args.path], args.graph, args.block)
    t = m["timing"]
    alg_bytes = block_bytes(w) if args.block else w.algorithmic_bytes()
    value_bytes = alg_bytes / (t["wall_ms_per_step"] * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value_bytes, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["wall_ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.DTYPE_NAMES[w.dtype],
        "data": "synthetic (seeded N(0,1) activations, N(0,1/d) weights, bf16 RNE)",
        "config": {"workload": w.name, "M": w.M, "d": w.d, "dff": w.dff,
                   "with_down": w.with_down, "path": PATH_NAMES[m["path"]],
                   "weight_copies": copies, "graph": bool(args.graph), "block": bool(args.block),
                   "algorithmic_bytes": alg_bytes,
                   "algorithmic_flops": w.algorithmic_flops()},
        "roofline": m["roofline"],
        "timing_ms": {k: round(v, 5) for k, v in t.items()},
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, m["runner"].inp, args.cpu_seconds)
    m["runner"].close()
    del m
    torch.cuda.empty_cache()
    if not args.no_variants and w.name == "decode8b_m1":
        # the same decode step with quantised weights (packed from the same
        # bf16 weights); reported beside the bf16 headline, never as it
        rec["quantized_decode"] = {}
        for name in ("decode8b_m1_fp8w", "decode8b_m1_mxfp4w"):
            q = wl.WORKLOADS[name]
            qcopies = max(1, -(-(1 << 30) // int(2 * q.d * q.dff * q.weight_bytes)))
            mq = measure(q, args.steps, args.warmup, qcopies)
            tq = mq["timing"]
            rec["quantized_decode"][name] = {
                "dtype": wl.DTYPE_NAMES[q.dtype],
                "value": round(q.algorithmic_bytes() / (tq["wall_ms_per_step"] * 1e-3) / 1e9, 1),
                "unit": "GB/s", "ms_per_step": round(tq["wall_ms_per_step"], 5),
                "algorithmic_bytes": q.algorithmic_bytes(), "roofline": mq["roofline"],
                "timing_ms": {k: round(v, 5) for k, v in tq.items()},
            }
            mq["runner"].close()
            del mq
            torch.cuda.empty_cache()
    if not args.no_prefill and w.name != "prefill8b_m4096":
        p = wl.WORKLOADS["prefill8b_m4096"]
        mp = measure(p, args.prefill_steps, args.prefill_warmup, 1)
        tp = mp["timing"]
        rec["prefill"] = {
            "workload": p.name, "M": p.M, "d": p.d, "dff": p.dff,
            "value": round(p.algorithmic_flops() / (tp["wall_ms_per_step"] * 1e-3) / 1e12, 1),
            "unit": "TFLOP/s", "ms_per_step": round(tp["wall_ms_per_step"], 4),
            "steps": args.prefill_steps, "warmup": args.prefill_warmup, "roofline": mp["roofline"],
            "timing_ms": {k: round(v, 5) for k, v in tp.items()},
        }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
