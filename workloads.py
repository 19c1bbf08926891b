"""Seeded synthetic inputs for the fused SwiGLU MLP, shared by the tests, the
bench and the smoke check.

This module holds no SwiGLU arithmetic: it only draws random numbers, rounds
them to the storage dtype, and describes the workload shapes.  Both the GPU
path and the CPU oracle consume exactly the arrays it returns.

Distributions follow the workloads of the pages (Qwen-2.5-style and 8B-class
MLP shapes, d_ff about 3.5 d, "Anatomie d'un transformeur sur GPU" §1.1
notation table): activations x ~ N(0, 1), gate/up weights ~ N(0, 1/d), down
weights ~ N(0, 1/d_ff).  Values are drawn in fp32 with NumPy's PCG64 and, for
bf16 workloads, rounded to bf16 with round-to-nearest-even on the host, so
every consumer sees identical bits.
"""
from __future__ import annotations

import dataclasses
import numpy as np

F32 = 0
BF16 = 1
FP8W = 2     # bf16 activations; weights packed as E4M3 codes (drawn here in bf16)
MXFP4W = 3   # bf16 activations; weights packed as MXFP4 (drawn here in bf16)
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8W: "bf16-fp8w", MXFP4W: "bf16-mxfp4w"}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark/parity shape: M rows of activations, d hidden, dff MLP."""
    cfg: int            # configuration number (1-based), used for seeds
    name: str
    M: int
    d: int
    dff: int
    dtype: int          # F32, BF16 or FP8W
    with_down: bool     # full MLP (gate/up + down projection) or up only
    m_max: int          # rows drawn for x; smaller M take the leading rows

    @property
    def elem_bytes(self) -> int:
        """Bytes per activation element (x, out, y)."""
        return 4 if self.dtype == F32 else 2

    @property
    def weight_bytes(self) -> float:
        """Bytes per stored weight (half a byte for MXFP4)."""
        return {FP8W: 1, MXFP4W: 0.5}.get(self.dtype, self.elem_bytes)

    def _weight_matrix_bytes(self, K: int, N: int) -> int:
        if self.dtype == FP8W:       # codes and one fp32 scale per column
            return K * N + 4 * N
        if self.dtype == MXFP4W:     # half-byte codes and one scale byte per 32
            return K * N // 2 + K * N // 32
        return K * N * self.elem_bytes

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move: weights once (with their scales when
        quantised), x once, output once."""
        s = self.elem_bytes
        b = 2 * self._weight_matrix_bytes(self.d, self.dff) + self.M * self.d * s
        if self.with_down:
            b += self._weight_matrix_bytes(self.dff, self.d) + self.M * self.d * s
        else:
            b += self.M * self.dff * s
        return b

    def algorithmic_flops(self) -> int:
        f = 4 * self.M * self.d * self.dff
        if self.with_down:
            f += 2 * self.M * self.dff * self.d
        return f


def _wl(cfg, name, M, d, dff, dtype, down, m_max):
    return Workload(cfg, name, M, d, dff, dtype, down, m_max)


# The five workload families, with every M they are run at.
WORKLOADS = {
    "tiny_decode_f32": _wl(1, "tiny_decode_f32", 1, 512, 2048, F32, False, 1),
    "decode8b_m1": _wl(2, "decode8b_m1", 1, 4096, 14336, BF16, False, 16),
    "decode8b_m4": _wl(2, "decode8b_m4", 4, 4096, 14336, BF16, False, 16),
    "decode8b_m8": _wl(2, "decode8b_m8", 8, 4096, 14336, BF16, False, 16),
    "decode8b_m16": _wl(2, "decode8b_m16", 16, 4096, 14336, BF16, False, 16),
    "mlp05b_m64": _wl(3, "mlp05b_m64", 64, 896, 4864, BF16, True, 64),
    "prefill8b_m4096": _wl(4, "prefill8b_m4096", 4096, 4096, 14336, BF16, False, 4096),
    "mlp72b_m16": _wl(5, "mlp72b_m16", 16, 8192, 29568, BF16, True, 2048),
    "mlp72b_m2048": _wl(5, "mlp72b_m2048", 2048, 8192, 29568, BF16, True, 2048),
    # batches between decode and prefill (the 8B-class prefill's first rows;
    # the 72B-class gate/up weights), on the many-rows path
    "prefill8b_m128": _wl(4, "prefill8b_m128", 128, 4096, 14336, BF16, False, 4096),
    "prefill8b_m256": _wl(4, "prefill8b_m256", 256, 4096, 14336, BF16, False, 4096),
    "prefill8b_m512": _wl(4, "prefill8b_m512", 512, 4096, 14336, BF16, False, 4096),
    "up72b_m512": _wl(5, "up72b_m512", 512, 8192, 29568, BF16, False, 2048),
    # the decode shapes with FP8 weights (same seeds, so the same bf16
    # weights before quantisation)
    "decode8b_m1_fp8w": _wl(2, "decode8b_m1_fp8w", 1, 4096, 14336, FP8W, False, 16),
    "decode8b_m16_fp8w": _wl(2, "decode8b_m16_fp8w", 16, 4096, 14336, FP8W, False, 16),
    "mlp72b_m16_fp8w": _wl(5, "mlp72b_m16_fp8w", 16, 8192, 29568, FP8W, True, 2048),
    "decode8b_m1_mxfp4w": _wl(2, "decode8b_m1_mxfp4w", 1, 4096, 14336, MXFP4W, False, 16),
    "decode8b_m16_mxfp4w": _wl(2, "decode8b_m16_mxfp4w", 16, 4096, 14336, MXFP4W, False, 16),
    "mlp72b_m16_mxfp4w": _wl(5, "mlp72b_m16_mxfp4w", 16, 8192, 29568, MXFP4W, True, 2048),
}

# tensor ids used in seeds: seed = 1000 * cfg + id
X_ID, WG_ID, WU_ID, WD_ID = 0, 1, 2, 3


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns
    the raw 16-bit patterns as uint16.  NaN inputs are not expected."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # finite inputs: u + 0x8000 stays below 2**32 (largest is 0xFF7FFFFF)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 patterns to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, shape, std: float) -> np.ndarray:
    """fp32 draws from N(0, std^2) with PCG64 seeded by `seed`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def to_storage(a32: np.ndarray, dtype: int) -> np.ndarray:
    """fp32 array -> storage array: float32 as is, or uint16 bf16 bits (also
    for FP8W, whose weights are quantised by the packer)."""
    if dtype == F32:
        return np.ascontiguousarray(a32, dtype=np.float32)
    return f32_to_bf16_bits(a32)


def make_inputs(w: Workload, with_down: bool | None = None, M: int | None = None):
    """Seeded inputs for workload `w`.

    Returns a dict with 'x' (M x d), 'wg' and 'wu' (d x dff) and, when the
    down projection is wanted, 'wd' (dff x d); all row-major, as float32
    arrays for F32 workloads or uint16 bf16 bit patterns for BF16 ones.
    """
    if with_down is None:
        with_down = w.with_down
    if M is None:
        M = w.M
    assert 0 <= M <= w.m_max
    base = 1000 * w.cfg
    out = {
        "x": to_storage(normal(base + X_ID, (w.m_max, w.d), 1.0)[:M], w.dtype),
        "wg": to_storage(normal(base + WG_ID, (w.d, w.dff), w.d ** -0.5), w.dtype),
        "wu": to_storage(normal(base + WU_ID, (w.d, w.dff), w.d ** -0.5), w.dtype),
    }
    if with_down:
        out["wd"] = to_storage(normal(base + WD_ID, (w.dff, w.d), w.dff ** -0.5), w.dtype)
    return out


def random_inputs(seed: int, M: int, d: int, dff: int, dtype: int, with_down=False,
                  x_std=1.0):
    """Inputs of an arbitrary shape with the workloads' distributions."""
    out = {
        "x": to_storage(normal(seed * 16 + X_ID, (M, d), x_std), dtype),
        "wg": to_storage(normal(seed * 16 + WG_ID, (d, dff), d ** -0.5), dtype),
        "wu": to_storage(normal(seed * 16 + WU_ID, (d, dff), d ** -0.5), dtype),
    }
    if with_down:
        out["wd"] = to_storage(normal(seed * 16 + WD_ID, (dff, d), dff ** -0.5), dtype)
    return out


def small_int(seed: int, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Small integers as fp32 (exact in bf16 too): used where every product
    and partial sum must be exact in fp32 whatever the summation order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def integer_inputs(seed: int, M: int, d: int, dff: int, dtype: int, with_down=False,
                   lo: int = -4, hi: int = 4):
    out = {
        "x": to_storage(small_int(seed * 16 + X_ID, (M, d), lo, hi), dtype),
        "wg": to_storage(small_int(seed * 16 + WG_ID, (d, dff), lo, hi), dtype),
        "wu": to_storage(small_int(seed * 16 + WU_ID, (d, dff), lo, hi), dtype),
    }
    if with_down:
        out["wd"] = to_storage(small_int(seed * 16 + WD_ID, (dff, d), lo, hi), dtype)
    return out


def one_hot_rows(M: int, d: int, ks, dtype: int) -> np.ndarray:
    """x whose row m is the unit vector e_{ks[m]}."""
    x = np.zeros((M, d), dtype=np.float32)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    return to_storage(x, dtype)
