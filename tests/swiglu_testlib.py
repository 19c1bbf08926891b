"""Helpers shared by the GPU tests: move seeded inputs to the device, call
the library through its C ABI, bring results back as fp64, and compare
them with the oracle under the tolerance rule
|gpu - ref| <= tol * (1 + |ref|) (tol 2e-2 for bf16 outputs, 1e-4 for fp32)."""
from __future__ import annotations

import sys

import numpy as np

import workloads as wl

# FP8 weights: bf16 outputs of fp32 sums over exactly widened codes, so the
# bf16 bar applies against the oracle's product with the same codes.
TOL = {wl.F32: 1e-4, wl.BF16: 2e-2, wl.FP8W: 2e-2, wl.MXFP4W: 2e-2}


def say(*args):
    """Print and flush: names the case before each GPU step."""
    print(*args, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU (no CPU fallback exists)"
    return torch


def dev(a: np.ndarray):
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t, dtype) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype != wl.F32:
        return wl.bf16_bits_to_f32(a.view(np.uint16)).astype(np.float64)
    return a.astype(np.float64)


def empty(shape, dtype):
    torch = torch_mod()
    return torch.empty(shape, dtype=torch.float32 if dtype == wl.F32 else torch.int16,
                       device="cuda")


def bytes_buf(n: int):
    torch = torch_mod()
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device="cuda")


def pack(inp: dict, d: int, dff: int, dtype: int):
    """Pack gate/up (and down, when present) on the GPU."""
    import gemv_gate_up_amd as sw
    wp = bytes_buf(sw.swiglu_packed_bytes(d, dff, dtype))
    sw.check(sw.swiglu_pack_weights(dev(inp["wg"]), dev(inp["wu"]), wp, d, dff, dtype),
             "swiglu_pack_weights")
    wdp = None
    if "wd" in inp:
        wdp = bytes_buf(sw.swiglu_down_packed_bytes(d, dff, dtype))
        sw.check(sw.swiglu_pack_down(dev(inp["wd"]), wdp, d, dff, dtype), "swiglu_pack_down")
    return wp, wdp


def run_up(x, wp, M, d, dff, dtype, path=0, sync=True):
    import gemv_gate_up_amd as sw
    nb = sw.swiglu_workspace_bytes_ex(M, d, dff, dtype, 0, path)
    ws = bytes_buf(nb) if nb else None
    out = empty((M, dff), dtype)
    sw.check(sw.swiglu_up_ex(x, wp, out, M, d, dff, dtype, ws, nb, None, path), "swiglu_up_ex")
    if sync:
        torch_mod().cuda.synchronize()
    return out


def run_mlp(x, wp, wdp, M, d, dff, dtype, path=0, sync=True):
    import gemv_gate_up_amd as sw
    nb = sw.swiglu_workspace_bytes_ex(M, d, dff, dtype, 1, path)
    ws = bytes_buf(nb)
    y = empty((M, d), dtype)
    sw.check(sw.mlp_forward_ex(x, wp, wdp, y, M, d, dff, dtype, ws, nb, None, path),
             "mlp_forward_ex")
    if sync:
        torch_mod().cuda.synchronize()
    return y


def compare(got: np.ndarray, ref: np.ndarray, tol: float) -> dict:
    """Element-wise check against the oracle plus the diagnostics of the
    accuracy reports (max error, share of elements off by more than 1%)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    scaled = err / (1.0 + np.abs(ref))
    big = np.abs(ref) > 1e-3
    rel = np.where(big, err / np.maximum(np.abs(ref), 1e-300), 0.0)
    worst = np.unravel_index(np.argmax(scaled), scaled.shape) if scaled.size else None
    return {
        "ok": bool(np.all(scaled <= tol)) and bool(np.all(np.isfinite(got))),
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_scaled": float(scaled.max()) if err.size else 0.0,
        "frac_rel_gt_1pct": float((rel > 0.01).mean()) if err.size else 0.0,
        "worst": tuple(int(i) for i in worst) if worst is not None else None,
    }


def assert_close(got, ref, dtype, what=""):
    st = compare(got, ref, TOL[dtype])
    assert st["ok"], "%s: %s" % (what, st)
    return st
