#!/usr/bin/env python3
"""Benchmark of the fused SwiGLU MLP hot path on one MI355X.

One step = one call of the hot path (swiglu_up, or mlp_forward for the
workloads with the down projection) through the C ABI, on inputs already
resident in HBM.  The JSON line's headline is the 8B-class decode step
(M = 1, d = 4096, d_ff = 14336, bf16) in HBM GB/s of algorithmic traffic
(both weight matrices once, x once, the output once).  The same line carries
every workload configuration under "configs" (and the quantised-weight decode
variants under "quantized_decode"), each with its step time, roofline,
sampled accuracy against the CPU oracle and the oracle's own time on the
host cores.

Weights rotate through a ring of copies (>= 1 GiB in total; one copy when a
copy is larger) so that the 256 MB Infinity Cache cannot serve a repeated
call: every timed call streams its weights from HBM.

Between workloads (never inside a timed region) the bench launches a tiny
fill kernel as a marker, three per workload (before set-up, before the first
step, after the last), so that a rocprofv3 trace or counter run of this
script can be cut into workloads; `--summarize DIR` turns such runs into the
summaries under profiles/.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only A,B]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
BF16_PEAK_MHZ = 2400.0         # the graphics clock that peak assumes
METRIC = "fused SwiGLU MLP: HBM GB/s at M=1 decode; bf16 TFLOP/s at M=4096 prefill"
HEADLINE = "decode8b_m1"
# the workload configurations, in run order
CONFIGS = ["tiny_decode_f32", "decode8b_m1", "decode8b_m4", "decode8b_m8", "decode8b_m16",
           "mlp05b_m64", "prefill8b_m4096", "mlp72b_m16", "mlp72b_m2048"]
QUANT_CONFIGS = ["decode8b_m1_fp8w", "decode8b_m1_mxfp4w", "decode8b_m16_fp8w",
                 "decode8b_m16_mxfp4w", "mlp72b_m16_fp8w", "mlp72b_m16_mxfp4w"]
RING_BYTES = 1 << 30
TOL = {wl.F32: 1e-4, wl.BF16: 2e-2, wl.FP8W: 2e-2, wl.MXFP4W: 2e-2}
MARKER_ELEMS = 4096
MARKER_NAME = "FillFunctor"    # torch's fill kernel: the markers' kernel name contains it

# sources each kernel family's code depends on (recorded counters are valid
# only for the sources they were taken on)
COMMON_SOURCES = ["geometry.h", "device_common.h", "launch.h", "api.hip"]
FAMILY_SOURCES = {
    "skinny_bf16_kernel": ["skinny.hip"], "skinny_f32_kernel": ["skinny.hip"],
    "skinny_f32m_kernel": ["skinny.hip"],
    "splitk_reduce_kernel": ["skinny.hip"], "wide_bf16_kernel": ["wide.hip", "wide_kernel.h"],
    "pack_act_kernel": ["pack.hip"], "rmsnorm_kernel": ["norm.hip"],
    "mlp_fused_kernel": ["fused.hip"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_family(name: str) -> str:
    """The kernel's unqualified name without template arguments."""
    base = name.split("(")[0].split("<")[0].strip()
    return base.split("::")[-1].split()[-1]


def source_file_hashes() -> dict:
    """sha256 of every kernel source file, as they are now."""
    out = {}
    d = os.path.join(ROOT, "gemv_gate_up_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            out[f] = hashlib.sha256(fh.read()).hexdigest()
    return out


def sources_hash(kernels, file_hashes=None) -> str:
    """Hash of the sources the given kernels depend on: the current files,
    or the per-file hashes a run recorded."""
    fh = file_hashes or source_file_hashes()
    files = list(COMMON_SOURCES)
    for k in kernels:
        for f in FAMILY_SOURCES.get(kernel_family(k), []):
            if f not in files:
                files.append(f)
    h = hashlib.sha256()
    for f in files:
        h.update(fh[f].encode())
    return h.hexdigest()[:16]


def traffic_record(workload: str):
    """The committed counter record of a workload's step, or None when it is
    missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("src_sha") != sources_hash(rec.get("kernels", [])):
        return None
    return rec


def weight_ring_copies(w: wl.Workload) -> int:
    one = 2 * w.d * w.dff * w.weight_bytes + (w.dff * w.d * w.weight_bytes if w.with_down else 0)
    return max(1, -(-RING_BYTES // int(one))) if one < RING_BYTES else 1


def hbm_bound(w: wl.Workload) -> bool:
    return w.algorithmic_flops() / w.algorithmic_bytes() < \
        BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)


def sample_rows(M: int):
    """Rows the accuracy check compares: every row up to 64, else one row in
    every 256-row tile (a different offset in each) and the last row."""
    if M <= 64:
        return None
    rows = {min(M - 1, t * 256 + (t * 37) % 256) for t in range(-(-M // 256))}
    rows.add(M - 1)
    return sorted(rows)


class Inputs:
    """Seeded inputs, shared by the workloads of one family (same seeds), and
    the oracle's quantised copies of their weights."""

    def __init__(self):
        self._fam, self._q = {}, {}

    def get(self, w: wl.Workload) -> dict:
        key = (w.cfg, w.with_down, w.dtype == wl.F32)
        if key not in self._fam:
            t0 = time.time()
            full = wl.Workload(w.cfg, w.name, w.m_max, w.d, w.dff,
                               wl.F32 if w.dtype == wl.F32 else wl.BF16, w.with_down, w.m_max)
            self._fam[key] = wl.make_inputs(full, M=w.m_max)
            log("inputs for %s generated in %.1fs" % (w.name, time.time() - t0))
        return self._fam[key]

    def weights_for_oracle(self, w: wl.Workload) -> dict:
        """Weights as the oracle takes them for this dtype: storage arrays,
        E4M3 (codes, scales) pairs, or dequantised MXFP4 fp64 arrays."""
        import oracle
        inp = self.get(w)
        names = ("wg", "wu", "wd") if w.with_down else ("wg", "wu")
        if w.dtype in (wl.F32, wl.BF16):
            return {k: inp[k] for k in names}
        key = (w.cfg, w.with_down, w.dtype)
        if key not in self._q:
            self._q = {}   # one quantised set at a time (MXFP4 keeps fp64 copies)
            if w.dtype == wl.FP8W:
                self._q[key] = {k: oracle.quantize_e4m3(inp[k]) for k in names}
            else:
                self._q[key] = {k: oracle.dequantize_mxfp4(*oracle.quantize_mxfp4(inp[k]))
                                for k in names}
        return self._q[key]


def oracle_call(w: wl.Workload, x: np.ndarray, wts: dict, rows=None, nthreads=0):
    """The oracle's result of the workload's step on x (fp64)."""
    import oracle
    if w.dtype == wl.FP8W:
        if w.with_down:
            return oracle.mlp_fp8w(x, *wts["wg"], *wts["wu"], *wts["wd"], rows=rows,
                                   nthreads=nthreads)
        return oracle.swiglu_fp8w(x, *wts["wg"], *wts["wu"], rows=rows, nthreads=nthreads)
    if w.dtype == wl.MXFP4W:
        x = oracle.to_double(x)
    if w.with_down:
        return oracle.mlp(x, wts["wg"], wts["wu"], wts["wd"], rows=rows, nthreads=nthreads)
    return oracle.swiglu(x, wts["wg"], wts["wu"], rows=rows, nthreads=nthreads)


def marker():
    """A tiny fill kernel that separates workloads in a trace or counter run."""
    import torch
    torch.empty(MARKER_ELEMS, dtype=torch.float32, device="cuda").fill_(1.0)


class Runner:
    """Device buffers and the C-ABI call for one workload."""

    def __init__(self, w: wl.Workload, inp: dict, copies: int, path: int = 0,
                 graph: bool = False, block: bool = False):
        import torch
        import gemv_gate_up_amd as sw
        self.torch, self.sw, self.w = torch, sw, w
        tdt = torch.float32 if w.dtype == wl.F32 else torch.int16

        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to("cuda")

        self.x = dev(inp["x"][:w.M])
        wp = torch.empty(sw.swiglu_packed_bytes(w.d, w.dff, w.dtype), dtype=torch.uint8,
                         device="cuda")
        sw.check(sw.swiglu_pack_weights(dev(inp["wg"]), dev(inp["wu"]), wp, w.d, w.dff,
                                        w.dtype), "pack")
        self.wps = [wp] + [wp.clone() for _ in range(copies - 1)]
        self.wdps = [None] * copies
        if w.with_down:
            wdp = torch.empty(sw.swiglu_down_packed_bytes(w.d, w.dff, w.dtype), dtype=torch.uint8,
                              device="cuda")
            sw.check(sw.swiglu_pack_down(dev(inp["wd"]), wdp, w.d, w.dff, w.dtype), "pack")
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
        elif w.with_down:
            rc = sw._lib.mlp_forward_ex(xp, wpp, wdpp, self.out.data_ptr(), w.M, w.d, w.dff,
                                        w.dtype, self.ws.data_ptr(), self.ws_bytes, self.sh,
                                        self.req_path)
        else:
            rc = sw._lib.swiglu_up_ex(xp, wpp, self.out.data_ptr(), w.M, w.d, w.dff, w.dtype,
                                      self.ws.data_ptr(), self.ws_bytes, self.sh, self.req_path)
        if rc != 0:
            raise RuntimeError("step failed: %s" % sw.swiglu_status_string(rc))

    def time(self, steps: int, warmup: int, window=None) -> dict:
        """K back-to-back steps between two synchronisations: the host clock
        gives the step rate, and a pair of HIP events recorded on the launch
        stream around the same K steps gives the device time per step.
        `window` (a context manager) is entered and left around them."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        if window is not None:
            window.__enter__()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(self.stream)
        for i in range(steps):
            self.step(warmup + i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if window is not None:
            window.__exit__(None, None, None)
        return {"wall_ms_per_step": (t1 - t0) * 1e3 / steps,
                "event_ms_per_step": e0.elapsed_time(e1) / steps}

    def result(self, rows=None) -> np.ndarray:
        """The last step's output (all weight copies are equal) as fp64."""
        o = self.out if rows is None else self.out[rows]
        a = o.cpu().numpy()
        if self.w.dtype != wl.F32:
            return wl.bf16_bits_to_f32(a.view(np.uint16)).astype(np.float64)
        return a.astype(np.float64)


PATHS = {"auto": 0, "skinny": 1, "wide": 2, "phased": 3, "fused": 4}
PATH_NAMES = {1: "skinny", 2: "wide", 3: "wide-phased", 4: "fused-down"}


def dominant_kernel(w: wl.Workload, path: int) -> str:
    if path == 4:
        return "mlp_fused_kernel"
    if path in (2, 3):
        return "wide_bf16_kernel"
    if w.dtype == wl.F32:   # the VALU kernel up to two rows, the matrix unit above
        return "skinny_f32_kernel" if w.M <= 2 else "skinny_f32m_kernel"
    return "skinny_bf16_kernel"


def block_bytes(w: wl.Workload) -> int:
    """Algorithmic bytes of the MLP block: the MLP's, plus gamma and bias
    (r is the MLP's x, out its y)."""
    return w.algorithmic_bytes() + 2 * w.d * w.elem_bytes


def max_ulps(err: np.ndarray, ref: np.ndarray, mant_bits: int) -> float:
    """Largest error in units in the last place of the reference, at an output
    precision of `mant_bits` explicit mantissa bits (7 for bf16, 23 for fp32);
    references below the smallest normal fp32 are left out."""
    a = np.abs(ref)
    normal = a >= 2.0 ** -126
    if not normal.any():
        return 0.0
    ulp = np.exp2(np.floor(np.log2(a[normal])) - mant_bits)
    return float((err[normal] / ulp).max())


def accuracy(got: np.ndarray, ref: np.ndarray, tol: float, what: str, dot_scale=None,
             mant_bits: int = 7) -> dict:
    """Pass/fail under |gpu - ref| <= tol (1 + |ref|), with the diagnostics:
    max error, max scaled error, the share of elements off by more than 1% of
    |ref| (elements with |ref| > 1e-3), the largest error in ulps of the
    reference, and (given dot_scale, the |a|.|b| scale of each output's sums)
    the largest error against that scale."""
    err = np.abs(got - ref)
    scaled = err / (1.0 + np.abs(ref))
    big = np.abs(ref) > 1e-3
    rel = np.where(big, err / np.maximum(np.abs(ref), 1e-300), 0.0)
    out = {"checked": what, "elements": int(got.size), "tol": tol,
           "ok": bool(np.all(np.isfinite(got)) and np.all(scaled <= tol)),
           "max_abs": float(err.max()), "max_scaled": float(scaled.max()),
           "frac_rel_gt_1pct": float((rel > 0.01).sum() / max(1, big.sum())),
           "max_ulps": max_ulps(err, ref, mant_bits)}
    if dot_scale is not None:
        pos = dot_scale > 0
        out["max_err_over_dot_scale"] = float((err[pos] / dot_scale[pos]).max()) if pos.any() else 0.0
    return out


def _abs_storage(a: np.ndarray) -> np.ndarray:
    """|a| in the same storage: bf16 bit patterns lose their sign bit."""
    if a.dtype == np.uint16:
        return a & np.uint16(0x7FFF)
    return np.abs(a)


_E4M3_TABLE = []


def _e4m3_table() -> np.ndarray:
    """The 256 E4M3 code values (the oracle's decoder), built once."""
    if not _E4M3_TABLE:
        import oracle
        _E4M3_TABLE.append(np.array([oracle.e4m3_to_double(c) for c in range(256)],
                                    dtype=np.float32))
    return _E4M3_TABLE[0]


def _as_f32(a) -> np.ndarray:
    """A matrix's values as float32: bf16 bit patterns widened (exact), fp32
    or fp64 arrays, or E4M3 (codes, per-column scales) pairs decoded."""
    if isinstance(a, tuple):
        codes, scales = a
        return _e4m3_table()[codes] * scales[None, :]
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32, copy=False)


def _row_products(xr: np.ndarray, W, absolute: bool):
    """xr . W and, with `absolute`, |xr| . |W| (fp64 results), decoding W to
    float32 2048 of its rows at a time so no full-size copy is made."""
    K = W[0].shape[0] if isinstance(W, tuple) else np.asarray(W).shape[0]
    n = W[0].shape[1] if isinstance(W, tuple) else np.asarray(W).shape[1]
    out = np.zeros((xr.shape[0], n))
    aout = np.zeros((xr.shape[0], n)) if absolute else None
    for k0 in range(0, K, 2048):
        k1 = min(K, k0 + 2048)
        blk = _as_f32((W[0][k0:k1], W[1]) if isinstance(W, tuple) else np.asarray(W)[k0:k1])
        xs = xr[:, k0:k1].astype(np.float32)
        out += xs @ blk
        if absolute:
            aout += np.abs(xs) @ np.abs(blk)
    return out, aout


def dot_scale(w: wl.Workload, x: np.ndarray, wts: dict, rows) -> np.ndarray:
    """The error scale of each output's sums, the |a|.|b| rule of "Où part le
    temps d'un token" (section on the narrow-matrix kernel) carried through
    the step, for the given rows of x: for out = silu(g) u,
    |d out/d g| sum|x||wg| + |d out/d u| sum|x||wu|; for y = out . Wd, the
    sum over d_ff of |out||wd|.  A diagnostic of the size of the rounding a
    correct fp32-accumulated result can show, computed in float32 from the
    weights as stored (quantised weights decoded), not a reference value."""
    xa = np.asarray(x)
    xr = _as_f32(xa if rows is None else xa[list(rows)]).astype(np.float64)
    down = w.with_down
    g, sg = _row_products(xr, wts["wg"], not down)
    u, su = _row_products(xr, wts["wu"], not down)
    sig = np.where(g >= 0, 1.0 / (1.0 + np.exp(-np.abs(g))),
                   np.exp(-np.abs(g)) / (1.0 + np.exp(-np.abs(g))))
    if down:
        _, sy = _row_products(np.abs(g * sig * u), wts["wd"], True)
        return sy
    return np.abs(u * sig * (1.0 + g * (1.0 - sig))) * sg + np.abs(g * sig) * su


def scale_rows(rows, M: int):
    """The rows the |a|.|b| diagnostic covers: the first and last of those
    checked (at most two, to keep the 72B-class weights' extra passes short)."""
    r = list(range(M)) if rows is None else list(rows)
    return sorted({r[0], r[-1]})


def cpu_baseline(w: wl.Workload, inputs: Inputs, budget_s: float, nthreads: int) -> dict:
    """The oracle, as it stands, on `nthreads` host cores: the workload's full
    step repeated for about budget_s (at least once); above 64 rows a
    contiguous block of 16 rows is timed instead and scaled linearly to M.
    Reported in the workload's unit."""
    inp = inputs.get(w)
    wts = inputs.weights_for_oracle(w)
    rows_timed = w.M if w.M <= 64 else 16
    x = inp["x"][:rows_timed]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle_call(w, x, wts, nthreads=nthreads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per_call = el / reps * (w.M / rows_timed)
    if hbm_bound(w):
        value, unit = w.algorithmic_bytes() / per_call / 1e9, "GB/s"
    else:
        value, unit = w.algorithmic_flops() / per_call / 1e12, "TFLOP/s"
    if rows_timed == w.M:
        sample = "%d full %s call(s) (M=%d, d=%d, dff=%d) in %.1f s wall, fp64" % (
            reps, w.name, w.M, w.d, w.dff, el)
    else:
        sample = ("%d call(s) on rows 0-%d of %s (d=%d, dff=%d) in %.1f s wall, fp64, "
                  "scaled linearly to M=%d" % (reps, rows_timed - 1, w.name, w.d, w.dff, el, w.M))
    return {"value": round(value, 4), "unit": unit, "cores": nthreads, "kind": "oracle",
            "sample": sample, "ms_per_call": round(per_call * 1e3, 3)}


def measure(w: wl.Workload, inputs: Inputs, steps: int, warmup: int, copies: int,
            path: int = 0, graph: bool = False, block: bool = False,
            check: bool = True, window=None, markers: bool = True,
            read_ceilings: bool = True) -> dict:
    """Times one workload; returns its record (and the runner, closed)."""
    mark = marker if markers else (lambda: None)
    mark()
    r = Runner(w, inputs.get(w), copies, path, graph, block)
    mark()
    t = r.time(steps, warmup, window)
    mark()
    bytes_alg = block_bytes(w) if block else w.algorithmic_bytes()
    flops_alg = w.algorithmic_flops()
    ms = t["event_ms_per_step"]
    kern = dominant_kernel(w, r.path)
    if hbm_bound(w):
        achieved = bytes_alg / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        value, unit = bytes_alg / (t["wall_ms_per_step"] * 1e-3) / 1e9, "GB/s"
    else:
        achieved = flops_alg / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
        value, unit = flops_alg / (t["wall_ms_per_step"] * 1e-3) / 1e12, "TFLOP/s"
    # recorded counters are for the dispatcher's own path with the reported workspace
    rec = traffic_record(w.name) if not (path or graph or block) else None
    roof["traffic"] = rec["hbm_bytes_per_step"] if rec else None
    roof["kernel"] = kern
    roof["step_kernels"] = rec["kernels"] if rec else None
    roof["event_ms_per_step"] = round(ms, 5)
    if hbm_bound(w) and read_ceilings:
        rc = read_ceiling(bytes_alg)
        roof["read_ceiling"] = rc
        roof["frac_of_read_ceiling"] = round(achieved / rc["gbps"], 4)
    out = {"workload": w.name, "M": w.M, "d": w.d, "dff": w.dff,
           "dtype": wl.DTYPE_NAMES[w.dtype], "with_down": w.with_down,
           "path": PATH_NAMES[r.path], "weight_copies": copies, "steps": steps, "warmup": warmup,
           "value": round(value, 3 if unit == "TFLOP/s" else 1), "unit": unit,
           "ms_per_step": round(t["wall_ms_per_step"], 5),
           "algorithmic_bytes": bytes_alg, "algorithmic_flops": flops_alg,
           "roofline": roof, "timing_ms": {k: round(v, 5) for k, v in t.items()}}
    if check and not block:
        rows = sample_rows(w.M)
        got = r.result(rows)
        inp = inputs.get(w)
        wts = inputs.weights_for_oracle(w)
        ref = oracle_call(w, inp["x"][:w.M], wts, rows=rows)
        what = ("every output" if rows is None else
                "%d whole rows (one per 256-row tile and the last)" % len(rows))
        acc = accuracy(got, ref, TOL[w.dtype], what, None, 23 if w.dtype == wl.F32 else 7)
        srows = scale_rows(rows, w.M)
        pos = [i for i, r in enumerate(list(range(w.M)) if rows is None else list(rows))
               if r in srows]
        sc = dot_scale(w, inp["x"][:w.M], wts, srows)
        err = np.abs(got[pos] - ref[pos])
        ok = sc > 0
        acc["max_err_over_dot_scale"] = float((err[ok] / sc[ok]).max()) if ok.any() else 0.0
        # ulps where the sum did not cancel to well below its terms' scale
        cond = np.abs(ref[pos]) >= 0.01 * sc
        acc["max_ulps_well_conditioned"] = max_ulps(err[cond], ref[pos][cond],
                                                    23 if w.dtype == wl.F32 else 7)
        acc["dot_scale_rows"] = srows
        out["accuracy"] = acc
    r.close()
    return out


class PowerSampler:
    """Samples the board's socket power and graphics clocks with `amd-smi
    metric -p -c` from a background thread while the timed steps run (after
    the warmup); a sample counts when it falls inside [start + skip, stop]."""

    CMD = ["amd-smi", "metric", "-p", "-c"]

    def __init__(self, skip_s: float = 0.5, period_s: float = 0.25):
        import threading
        self.skip_s, self.period_s = skip_s, period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)
        self.t0 = self.t1 = None

    def _read(self):
        import re
        import subprocess
        try:
            txt = subprocess.run(self.CMD, capture_output=True, text=True, timeout=10).stdout
        except (OSError, subprocess.TimeoutExpired):
            return None
        pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", txt)
        clks = [float(c) for c in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", txt)]
        if not pw or not clks:
            return None
        return float(pw.group(1)), clks

    def _loop(self):
        while not self._stop.is_set():
            t = time.perf_counter()
            r = self._read()
            if r is not None:
                self.samples.append((t, r[0], r[1]))
            self._stop.wait(self.period_s)

    def __enter__(self):
        self.t0 = time.perf_counter()
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self.t1 = time.perf_counter()
        self._stop.set()
        self._thread.join()

    def summary(self) -> dict:
        keep = [s for s in self.samples if self.t0 + self.skip_s <= s[0] <= self.t1]
        out = {"command": " ".join(self.CMD), "samples": len(keep),
               "window_s": round(self.t1 - self.t0 - self.skip_s, 2)}
        if keep:
            out["socket_w_mean"] = round(statistics.mean(s[1] for s in keep), 1)
            out["socket_w_max"] = round(max(s[1] for s in keep), 1)
            clk = [statistics.mean(s[2]) for s in keep]
            out["gfx_mhz_mean"] = round(statistics.mean(clk), 1)
            out["gfx_mhz_min"] = round(min(min(s[2]) for s in keep), 1)
            out["gfx_mhz_max"] = round(max(max(s[2]) for s in keep), 1)
        return out


# The matrix-bound workload whose board power and clock the default run
# records: under it the board sits at its power limit and the clock drops.
POWER_WORKLOAD = "prefill8b_m4096"


def power_window(w: wl.Workload, inputs: Inputs, rec: dict, seconds: float, copies: int) -> dict:
    """Runs the workload again for about `seconds` of timed steps (untimed
    for the record) while sampling board power and clocks; adds the
    fraction of the bf16 peak at the mean sampled clock."""
    ms = rec["roofline"]["event_ms_per_step"]
    steps = max(20, int(seconds * 1e3 / ms))
    sampler = PowerSampler(skip_s=1.0)   # the board's power control settles within about a second
    # no markers: a trace's per-workload segments stay as the timed run cut them
    measure(w, inputs, steps, 20, copies, check=False, window=sampler, markers=False,
            read_ceilings=False)
    out = sampler.summary()
    out["steps"] = steps
    if out.get("gfx_mhz_mean"):
        at_clock = BF16_PEAK_TFLOPS * out["gfx_mhz_mean"] / BF16_PEAK_MHZ
        out["peak_at_clock_tflops"] = round(at_clock, 1)
        out["frac_at_clock"] = round(rec["roofline"]["achieved"] / at_clock, 4)
    return out


_PROBE = []
_READ_CEILINGS = {}


def _probe_lib():
    """The measurement-aid library built beside libswiglu.so (a plain read,
    device attributes); loaded once."""
    if not _PROBE:
        import ctypes
        lib = ctypes.CDLL(os.path.join(ROOT, "gemv_gate_up_amd", "libswiglu_probe.so"))
        lib.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.probe_device.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
        _PROBE.append(lib)
    return _PROBE[0]


def read_ceiling(nbytes: int) -> dict:
    """The best time of a plain streaming read of nbytes (the probe library's
    grid-stride kernel: 512-4096 workgroups, 4-16 nontemporal 16-byte loads
    in flight per thread) over a ring of copies of at least 1 GiB, so that
    the Infinity Cache serves none of it: the HBM rate a kernel can reach at
    this size on this board.  Cached per size."""
    nb = int(nbytes) // 16 * 16
    if nb in _READ_CEILINGS:
        return _READ_CEILINGS[nb]
    import torch
    lib = _probe_lib()
    copies = max(2, -(-(1 << 30) // nb))
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    stream = torch.cuda.current_stream()
    best = None
    for grid in (512, 1024, 2048, 4096):
        sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
        for u in (4, 8, 16):
            def go(i):
                rc = lib.probe_read(bufs[i % copies].data_ptr(), nb, sink.data_ptr(), grid, u,
                                    stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError("probe_read failed (%d)" % rc)
            for i in range(10):
                go(i)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            n = 30
            e0.record(stream)
            for i in range(n):
                go(i)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / n * 1e3
            if best is None or us < best[0]:
                best = (us, grid, u)
    del bufs
    torch.cuda.empty_cache()
    rec = {"bytes": nb, "us": round(best[0], 3), "gbps": round(nb / best[0] / 1e3, 1),
           "grid": best[1], "loads_in_flight": best[2]}
    _READ_CEILINGS[nb] = rec
    return rec


def device_record() -> dict:
    """The device's compute units and maximum graphics clock (HIP device
    attributes) and the dense bf16 matrix peak they give: 4096 FLOPs per
    clock per CU."""
    import ctypes
    import torch
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    rc = _probe_lib().probe_device(ctypes.byref(cus), ctypes.byref(khz))
    if rc != 0:
        return {"error": rc}
    return {"name": torch.cuda.get_device_name(0), "compute_units": cus.value,
            "max_clock_mhz": khz.value / 1000.0,
            "bf16_peak_tflops": round(cus.value * 4096 * khz.value * 1e3 / 1e12, 1)}


def run_order(only):
    """The default workloads in order, or those named (the default ones in
    their order, then any others as given)."""
    names = CONFIGS + QUANT_CONFIGS
    if not only:
        return names
    return [n for n in names if n in only] + [n for n in only if n not in names]


def probe(order) -> int:
    """Kernels for hardware-counter runs: a plain copy of known size (reads
    and writes exactly 1 GiB) to calibrate FETCH_SIZE / WRITE_SIZE, then
    a few steps of each workload as the bench runs them (with its markers);
    prints no timing."""
    import torch
    print(json.dumps({"probe_order": order, "src_files": source_file_hashes()}), flush=True)
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")   # no fill: a fill is a marker
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    inputs = Inputs()
    for name in order:
        w = wl.WORKLOADS[name]
        marker()
        r = Runner(w, inputs.get(w), weight_ring_copies(w))
        marker()
        for i in range(5):
            r.step(i)
        marker()
        torch.cuda.synchronize()
        r.close()
        del r
        torch.cuda.empty_cache()
    log("probe done")
    return 0


# ---------------------------------------------------------------- profiles
def _segments(names):
    """Cuts a dispatch sequence at the bench's markers: for each workload,
    the dispatches between its second and third marker (its steps)."""
    idx = [i for i, n in enumerate(names) if MARKER_NAME in n]
    if len(idx) % 3:
        raise ValueError("marker count %d is not a multiple of 3" % len(idx))
    return [(idx[3 * j + 1] + 1, idx[3 * j + 2]) for j in range(len(idx) // 3)]


def _step_kernels(names, nsteps):
    """Kernel names of one step, from a run of nsteps identical steps."""
    if not names or len(names) % nsteps:
        raise ValueError("%d dispatches do not split into %d steps" % (len(names), nsteps))
    k = len(names) // nsteps
    step = names[:k]
    if names != step * nsteps:
        raise ValueError("steps do not repeat the same kernels")
    return step


def _read_csv(pattern):
    files = glob.glob(pattern, recursive=True)
    if not files:
        raise FileNotFoundError(pattern)
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counter_per_step(rows, order, nsteps=5):
    """Per workload: (step kernel names, counter KiB per kernel of a step,
    averaged over the steps), plus the calibration copy's mean."""
    rows = sorted(rows, key=lambda x: int(x["Dispatch_Id"]))
    names = [r["Kernel_Name"] for r in rows]
    vals = [float(r["Counter_Value"]) for r in rows]
    cal = [v for n, v, r in zip(names, vals, rows)
           if "copyBuffer" in n and int(r["Grid_Size"]) == 131072][:3]
    if len(cal) != 3:
        raise ValueError("calibration copies not found")
    out = {}
    for name, (a, b) in zip(order, _segments(names)):
        step = _step_kernels(names[a:b], nsteps)
        k = len(step)
        per = [statistics.mean(vals[a + j::k][:nsteps]) for j in range(k)]
        out[name] = (step, per)
    return out, statistics.mean(cal)


# Extra counter passes (rocprofv3 --pmc of --probe, one directory each:
# d/pmc_<tag>/ with its stdout in d/pmc_<tag>.log), within one pass's limits
# (at most 8 SQ, 4 TCC, 2 GRBM counters)
PMC_PASSES = {
    "a": "MfmaUtil SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY "
         "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_MFMA",
    "b": "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_DRAM_sum SQ_LDS_BANK_CONFLICT "
         "SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM "
         "GRBM_GUI_ACTIVE",
}


def _multi_counter_per_step(rows, order, nsteps=5):
    """Like _counter_per_step for a pass with several counters: per workload,
    (step kernel names, [{counter: mean over the steps} per kernel])."""
    by_disp = {}
    for r in rows:
        e = by_disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "c": {}})
        e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [by_disp[k] for k in sorted(by_disp)]
    names = [e["name"] for e in disp]
    out = {}
    for name, (a, b) in zip(order, _segments(names)):
        step = _step_kernels(names[a:b], nsteps)
        k = len(step)
        per = []
        for j in range(k):
            runs = disp[a + j:b:k][:nsteps]
            per.append({c: statistics.mean(x["c"][c] for x in runs) for c in runs[0]["c"]})
        out[name] = (step, per)
    return out


def _counter_section(name, step, passes) -> list:
    """Markdown lines with the extra counter passes' values for one workload."""
    lines = []
    for tag, data in sorted(passes.items()):
        if name not in data:
            continue
        pstep, per = data[name]
        if [kernel_family(s) for s in pstep] != [kernel_family(s) for s in step]:
            raise ValueError("%s: pass %s launched other kernels" % (name, tag))
        cols = sorted(per[0])
        lines += ["", "Counters (pass %s, mean of 5 probe steps per launch): "
                  "`cd /tmp && rocprofv3 --pmc %s --output-format csv -d <out>/pmc_%s -o probe -- "
                  "python3 <repo>/bench.py --probe --only <workloads>`" % (tag, PMC_PASSES[tag], tag),
                  "", "| # | kernel | " + " | ".join(cols) + " |",
                  "|---|---|" + "---|" * len(cols)]
        for j, s in enumerate(pstep):
            lines.append("| %d | %s | " % (j + 1, kernel_family(s)) +
                         " | ".join("%.4g" % per[j][c] for c in cols) + " |")
        derived = []
        for j, s in enumerate(pstep):
            c = per[j]
            parts = []
            if "SQ_WAIT_INST_ANY" in c and c.get("SQ_WAVE_CYCLES"):
                parts.append("waves waiting on an instruction's operands %.1f%% of their "
                             "cycles" % (100 * c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]))
            if "SQ_WAIT_ANY" in c and c.get("SQ_WAVE_CYCLES"):
                parts.append("waiting on anything %.1f%%" %
                             (100 * c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]))
            if c.get("TCC_HIT_sum", 0) + c.get("TCC_MISS_sum", 0) > 0:
                parts.append("L2 hit rate %.1f%%" % (100 * c["TCC_HIT_sum"] /
                                                     (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])))
            if c.get("TCC_EA0_RDREQ_sum"):
                parts.append("%.1f%% of L2 read requests to memory marked DRAM" %
                             (100 * c.get("TCC_EA0_RDREQ_DRAM_sum", 0) / c["TCC_EA0_RDREQ_sum"]))
            if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_LDS_IDX_ACTIVE"):
                parts.append("LDS bank-conflict cycles %.2f%% of LDS active cycles" %
                             (100 * c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]))
            if parts:
                derived.append("* %s (%d): %s." % (kernel_family(s), j + 1, "; ".join(parts)))
        if derived:
            lines += [""] + derived
    return lines


def summarize(d: str) -> int:
    """Writes profiles/traffic_<workload>.json and profiles/<kernel>-<workload>.md
    from a directory of rocprofv3 runs of this script:
      d/trace/**/*kernel_trace.csv   --kernel-trace --stats of the default bench run
      d/trace_bench.log              that run's stdout (the JSON line)
      d/fetch/**/*counter_collection.csv, d/write/...   --pmc FETCH_SIZE / WRITE_SIZE of --probe
    """
    bench_line = json.loads([ln for ln in open(os.path.join(d, "trace_bench.log"))
                             if ln.startswith("{")][-1])
    order = bench_line["order"]
    recs = dict(bench_line["configs"])
    recs.update(bench_line.get("quantized_decode", {}))
    tr = _read_csv(os.path.join(d, "trace", "**", "*kernel_trace.csv"))
    tr.sort(key=lambda x: int(x["Start_Timestamp"]))
    tnames = [x["Kernel_Name"] for x in tr]
    fetch_rows = _read_csv(os.path.join(d, "fetch", "**", "*counter_collection.csv"))
    write_rows = _read_csv(os.path.join(d, "write", "**", "*counter_collection.csv"))
    plog = json.loads([ln for ln in open(os.path.join(d, "fetch.log"))
                       if ln.startswith('{"probe_order"')][0])
    porder = plog["probe_order"]
    # every run must have been made on the same sources; the records carry
    # the hash of those sources, not of the files as they are now
    src = bench_line["src_files"]
    for other in [plog] + [json.loads([ln for ln in open(os.path.join(d, f)) if
                                       ln.startswith('{"probe_order"')][0])
                           for f in ("write.log",) + tuple(
                               os.path.basename(p) + ".log"
                               for p in glob.glob(os.path.join(d, "pmc_*")) if os.path.isdir(p))]:
        if other.get("src_files") != src:
            raise ValueError("the runs in %s were made on different sources" % d)
    fetch, fcal = _counter_per_step(fetch_rows, porder)
    write, wcal = _counter_per_step(write_rows, porder)
    ff, wf = (1 << 20) / fcal, (1 << 20) / wcal
    passes = {}
    for pdir in sorted(glob.glob(os.path.join(d, "pmc_*"))):
        if not os.path.isdir(pdir):
            continue
        tag = os.path.basename(pdir)[4:]
        plog = [ln for ln in open(pdir + ".log") if ln.startswith('{"probe_order"')]
        passes[tag] = _multi_counter_per_step(
            _read_csv(os.path.join(pdir, "**", "*counter_collection.csv")),
            json.loads(plog[0])["probe_order"])
    trace_cmd = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace "
                 "-o bench -- python3 <repo>/bench.py --no-cpu --power-seconds 0")
    pmc_cmd = ("cd /tmp && rocprofv3 --pmc %s --output-format csv -d <out>/%s -o probe -- "
               "python3 <repo>/bench.py --probe")
    for name, (a, b) in zip(order, _segments(tnames)):
        rec = recs[name]
        steps = rec["steps"]
        disp = tr[a:b]
        step = _step_kernels([x["Kernel_Name"] for x in disp], steps + rec["warmup"])
        k = len(step)
        timed = disp[len(disp) - k * steps:]
        durs = [[(int(x["End_Timestamp"]) - int(x["Start_Timestamp"])) for x in timed[j::k]]
                for j in range(k)]
        span = (int(timed[-1]["End_Timestamp"]) - int(timed[0]["Start_Timestamp"])) / steps
        fstep, fper = fetch[name]
        wstep, wper = write[name]
        if [kernel_family(s) for s in fstep] != [kernel_family(s) for s in step] or \
                [kernel_family(s) for s in wstep] != [kernel_family(s) for s in step]:
            raise ValueError("%s: the counter runs launched other kernels" % name)
        fb = [round(v * 1024 * ff) for v in fper]
        wb = [round(v * 1024 * wf) for v in wper]
        total = sum(fb) + sum(wb)
        alg = rec["algorithmic_bytes"]
        sha = sources_hash(step, src)
        traffic = {"workload": name, "src_sha": sha, "kernels": [kernel_family(s) for s in step],
                   "kernel_names": step, "fetch_factor": round(ff, 5), "write_factor": round(wf, 5),
                   "fetch_kib_raw": [round(v, 1) for v in fper],
                   "write_kib_raw": [round(v, 1) for v in wper],
                   "hbm_bytes_per_step": total, "algorithmic_bytes": alg,
                   "ratio": round(total / alg, 3)}
        with open(os.path.join(ROOT, "profiles", "traffic_%s.json" % name), "w") as f:
            json.dump(traffic, f, indent=1)
            f.write("\n")
        dom = rec["roofline"]["kernel"]
        rows = []
        for j, s in enumerate(step):
            dj = durs[j]
            rows.append("| %d | `%s` | %d | %.0f | %d | %d | %d | %d |" % (
                j + 1, s[:110], len(dj), statistics.mean(dj), min(dj), max(dj), fb[j], wb[j]))
        ksum = sum(statistics.mean(dj) for dj in durs) / 1e3
        rl = rec["roofline"]
        md = "\n".join([
            "# %s: %s (MI355X, gfx950)" % (name, ", ".join(kernel_family(s) for s in step)),
            "",
            "Kernel sources sha256[:16] = `%s` (bench.py `sources_hash` over this step's "
            "kernels). %s steps of M=%d, d=%d, dff=%d (%s, %s), %d timed after %d warmup, "
            "weights rotated over %d copies." % (sha, "MLP" if rec["with_down"] else "swiglu_up",
                                                 rec["M"], rec["d"], rec["dff"], rec["dtype"],
                                                 rec["path"], steps, rec["warmup"],
                                                 rec["weight_copies"]),
            "",
            "Kernel trace: `%s`" % trace_cmd,
            "",
            "HBM counters: `%s` and the same with `WRITE_SIZE` (`<out>/write`)."
            % (pmc_cmd % ("FETCH_SIZE", "fetch")),
            "",
            "Per kernel of one step, over the %d timed steps only (trace), and its HBM bytes per "
            "launch (counters, mean of 5 probe steps; fetch x %.4f, write x %.4f from a 1 GiB "
            "copy):" % (steps, ff, wf),
            "",
            "| # | kernel | launches | average ns | min ns | max ns | fetch B | write B |",
            "|---|---|---|---|---|---|---|---|",
        ] + rows + [
            "",
            "Sum of the kernel averages: %.2f us per step; first start to last end over the "
            "timed steps: %.2f us per step. bench.py in the same run (HIP events on the launch "
            "stream around the same steps): %.2f us per step, roofline frac %.4f of %s %s." % (
                ksum, span / 1e3, rl["event_ms_per_step"] * 1e3, rl["frac"], rl["peak"],
                rl["unit"]),
        ] + ([
            "",
            "In this traced run the span and the events include gaps between the launches that "
            "the tracer adds (%.2f us per step beyond the kernels' own time); the kernel "
            "averages are the figures to compare with an untraced run's events." % (
                span / 1e3 - ksum)] if span / 1e3 > 1.1 * ksum else []) + [
            "",
            "HBM traffic per step: fetch %d B + write %d B = **%d B** against %d algorithmic "
            "bytes (ratio %.2f)." % (sum(fb), sum(wb), total, alg, total / alg)]
            + _counter_section(name, step, passes) + [""])
        fn = os.path.join(ROOT, "profiles", "%s-%s.md" % (dom, name))
        with open(fn, "w") as f:
            f.write(md)
        log("wrote", fn)
    return 0


# ---------------------------------------------------------------- main
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200,
                    help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config-steps", type=int, default=100,
                    help="timed steps of the other decode-regime workloads (at least --steps)")
    ap.add_argument("--prefill-steps", type=int, default=20,
                    help="timed steps of the compute-bound workloads")
    ap.add_argument("--prefill-warmup", type=int, default=40,
                    help="their untimed steps first: the clock needs ~30 ms of matrix work "
                         "to settle")
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(wl.WORKLOADS),
                    help="headline workload (the configs are still all run unless --only)")
    ap.add_argument("--only", default="",
                    help="comma-separated workloads to run besides the headline (default: all)")
    ap.add_argument("--block", action="store_true",
                    help="time the MLP block (RMSNorm, MLP, bias and residual) on the headline "
                         "workload, which needs the down projection; no configs")
    ap.add_argument("--graph", action="store_true",
                    help="replay recorded calls (HIP graphs) on the headline workload; no configs")
    ap.add_argument("--power", action="store_true",
                    help="sample socket power and graphics clocks (amd-smi) while the headline "
                         "workload's timed steps run (pass --steps for a few seconds of work); "
                         "no configs")
    ap.add_argument("--power-seconds", type=float, default=4.0,
                    help="seconds of extra %s steps under the power sampler in the default "
                         "run (0: none)" % POWER_WORKLOAD)
    ap.add_argument("--path", default="auto", choices=sorted(PATHS),
                    help="force a kernel path for the headline workload; no configs")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="oracle time budget of the headline's CPU baseline")
    ap.add_argument("--config-cpu-seconds", type=float, default=1.5)
    ap.add_argument("--probe", action="store_true",
                    help="counter-collection run: a 1 GiB device copy (calibration), then a few "
                         "steps of every workload; prints no timing")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write profiles/ from rocprofv3 runs of this script in DIR (no GPU)")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args.summarize)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(one GPU's share of a sharded MLP is the same kernel at a smaller d_ff).",
              file=sys.stderr)
        return 2

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    only = [s for s in args.only.split(",") if s]
    for s in only:
        if s not in wl.WORKLOADS:
            ap.error("unknown workload %s" % s)
    order = run_order(only)
    if args.probe:
        return probe(order)
    import oracle
    cores = oracle.available_cores()
    inputs = Inputs()
    hw = wl.WORKLOADS[args.workload]
    special = args.block or args.graph or args.power or args.path != "auto"

    def steps_of(w):
        if w.name == hw.name:
            return args.steps, args.warmup
        if hbm_bound(w):
            return max(args.steps, args.config_steps), max(args.warmup, 20)
        return args.prefill_steps, args.prefill_warmup

    def run(w, headline=False):
        steps, warmup = steps_of(w)
        copies = weight_ring_copies(w)
        log("workload %s: %s, %d weight copies" % (w.name, w, copies))
        sampler = PowerSampler() if args.power and headline else None
        rec = measure(w, inputs, steps, warmup, copies,
                      PATHS[args.path] if headline else 0, args.graph and headline,
                      args.block and headline, check=not sampler, window=sampler)
        if sampler:
            rec["power"] = sampler.summary()
        elif w.name == POWER_WORKLOAD and not special and args.power_seconds > 0:
            rec["power"] = power_window(w, inputs, rec, args.power_seconds, copies)
        torch.cuda.empty_cache()
        if not args.no_cpu:
            budget = args.cpu_seconds if headline else args.config_cpu_seconds
            rec["cpu_baseline"] = cpu_baseline(w, inputs, budget, cores)
            if w.name in ("tiny_decode_f32", "decode8b_m1") and not special:
                rec["cpu_baseline"]["single_thread"] = cpu_baseline(w, inputs, 2.0, 1)
        return rec

    configs, quant = {}, {}
    run_names = [] if special else [n for n in order if n != hw.name]
    # the headline runs first when it is not one of the configs
    head = run(hw, headline=True)
    executed = [hw.name]
    for name in run_names:
        w = wl.WORKLOADS[name]
        (quant if name in QUANT_CONFIGS else configs)[name] = run(w)
        executed.append(name)
    if hw.name in CONFIGS and not special:
        configs[hw.name] = head
    elif hw.name in QUANT_CONFIGS and not special:
        quant[hw.name] = head
    headline_value = head["value"]
    rec = {
        "metric": METRIC,
        "value": headline_value,
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) activations, N(0,1/d) weights, bf16 RNE)",
        "config": {"workload": hw.name, "M": hw.M, "d": hw.d, "dff": hw.dff,
                   "with_down": hw.with_down, "path": head["path"],
                   "weight_copies": head["weight_copies"], "graph": bool(args.graph),
                   "block": bool(args.block), "algorithmic_bytes": head["algorithmic_bytes"],
                   "algorithmic_flops": head["algorithmic_flops"]},
        "roofline": head["roofline"],
        "timing_ms": head["timing_ms"],
    }
    if "accuracy" in head:
        rec["accuracy"] = head["accuracy"]
    if "power" in head:
        rec["power"] = head["power"]
    if "cpu_baseline" in head:
        rec["cpu_baseline"] = head["cpu_baseline"]
    if "prefill8b_m4096" in configs:
        p = configs["prefill8b_m4096"]
        rec["prefill"] = {k: p[k] for k in ("workload", "M", "d", "dff", "value", "unit",
                                            "ms_per_step", "steps", "warmup", "roofline",
                                            "power") if k in p}
    if configs:
        rec["configs"] = configs
    if quant:
        rec["quantized_decode"] = quant
    rec["device"] = device_record()
    rec["order"] = executed
    rec["src_files"] = source_file_hashes()
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
