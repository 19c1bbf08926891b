"""Python binding of libswiglu.so, the MI355X (gfx950) fused SwiGLU MLP
library.  Argument marshalling only: every step of the computation runs in
the library's HIP kernels.

The functions carry the C names of include/swiglu.h and return its integer
status codes.  Pointer arguments accept a torch tensor (its data_ptr), an int
device address, or None.  `stream` accepts None (torch's current stream), a
torch.cuda.Stream, or a raw hipStream_t as int.

Importing this package raises ImportError if the library has not been built
(python gemv_gate_up_amd/build.py): there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswiglu.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "swiglu.h")

SWIGLU_F32 = 0
SWIGLU_BF16 = 1
SWIGLU_BF16_FP8W = 2
SWIGLU_BF16_MXFP4W = 3

SWIGLU_OK = 0
SWIGLU_ERR_INVALID_ARG = -1
SWIGLU_ERR_UNSUPPORTED = -2
SWIGLU_ERR_MISALIGNED = -3
SWIGLU_ERR_WORKSPACE = -4
SWIGLU_ERR_HIP = -5
SWIGLU_ERR_SCRATCH = -6
SWIGLU_SCRATCH_BYTES = 32 << 20

SWIGLU_PATH_AUTO = 0
SWIGLU_PATH_SKINNY = 1
SWIGLU_PATH_WIDE = 2
SWIGLU_PATH_WIDE_PHASED = 3
SWIGLU_PATH_FUSED_DOWN = 4


class SwigluError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s: %s (%d)" % (what or "swiglu", swiglu_status_string(status), status))


# One HIP runtime per process.  PyTorch's ROCm wheel ships its own
# libamdhip64 and links it under a name (libamdhip64.so) that differs from
# the one this library links (libamdhip64.so.7, found under /opt/rocm).  If
# this library were loaded first, importing torch afterwards would map a
# second runtime, and device pointers and streams from one runtime are not
# valid in the other.  Importing torch first makes the dynamic linker bind
# this library to the runtime already in the process (same soname).
try:
    import torch as _torch  # noqa: F401
except ImportError:   # a process without torch has only one runtime anyway
    _torch = None

if not os.path.exists(LIB_PATH):
    raise ImportError("libswiglu.so is not built; run `python gemv_gate_up_amd/build.py` "
                      "(expected at %s)" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

_i64, _sz, _vp, _int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
_SIGS = {
    "swiglu_status_string": (ctypes.c_char_p, [_int]),
    "swiglu_version": (_int, []),
    "swiglu_packed_bytes": (_sz, [_i64, _i64, _int]),
    "swiglu_down_packed_bytes": (_sz, [_i64, _i64, _int]),
    "swiglu_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _int]),
    "swiglu_workspace_bytes_ex": (_sz, [_i64, _i64, _i64, _int, _int, _int]),
    "swiglu_select_path": (_int, [_i64, _i64, _i64, _int]),
    "swiglu_pack_weights": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _vp]),
    "swiglu_pack_down": (_int, [_vp, _vp, _i64, _i64, _int, _vp]),
    "swiglu_up": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _sz, _vp]),
    "swiglu_up_ex": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _sz, _vp, _int]),
    "swiglu_up_noalloc": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _vp]),
    "mlp_forward": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _sz, _vp]),
    "mlp_forward_ex": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _sz, _vp, _int]),
    "swiglu_up_graph_create": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _sz, _int,
                                      ctypes.POINTER(_vp)]),
    "mlp_forward_graph_create": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _sz,
                                        _int, ctypes.POINTER(_vp)]),
    "mlp_block_graph_create": (_int, [_vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _i64, _i64,
                                      _i64, _int, _vp, _sz, _int, ctypes.POINTER(_vp)]),
    "swiglu_graph_launch": (_int, [_vp, _vp]),
    "mlp_block_workspace_bytes": (_sz, [_i64, _i64, _i64, _int]),
    "mlp_block_workspace_bytes_ex": (_sz, [_i64, _i64, _i64, _int, _int]),
    "mlp_block_forward": (_int, [_vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                 _int, _vp, _sz, _vp]),
    "mlp_block_forward_ex": (_int, [_vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _i64, _i64,
                                    _i64, _int, _vp, _sz, _vp, _int]),
    "swiglu_graph_destroy": (_int, [_vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def header_functions() -> list[str]:
    """Names of the functions include/swiglu.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "defined"})


def _ptr(p):
    if p is None:
        return None
    if isinstance(p, int):
        return p
    return p.data_ptr()


def _stream(s):
    if isinstance(s, int):
        return s
    import torch
    if s is None:
        s = torch.cuda.current_stream()
    return s.cuda_stream


def swiglu_status_string(status: int) -> str:
    return _lib.swiglu_status_string(status).decode()


def swiglu_version() -> int:
    return _lib.swiglu_version()


def swiglu_packed_bytes(d: int, dff: int, dtype: int) -> int:
    return _lib.swiglu_packed_bytes(d, dff, dtype)


def swiglu_down_packed_bytes(d: int, dff: int, dtype: int) -> int:
    return _lib.swiglu_down_packed_bytes(d, dff, dtype)


def swiglu_workspace_bytes(M: int, d: int, dff: int, dtype: int, with_down: int) -> int:
    return _lib.swiglu_workspace_bytes(M, d, dff, dtype, int(with_down))


def swiglu_workspace_bytes_ex(M, d, dff, dtype, with_down, path) -> int:
    return _lib.swiglu_workspace_bytes_ex(M, d, dff, dtype, int(with_down), path)


def swiglu_select_path(M: int, d: int, dff: int, dtype: int) -> int:
    return _lib.swiglu_select_path(M, d, dff, dtype)


def swiglu_pack_weights(Wgate, Wup, Wpacked, d, dff, dtype, stream=None) -> int:
    return _lib.swiglu_pack_weights(_ptr(Wgate), _ptr(Wup), _ptr(Wpacked), d, dff, dtype,
                                    _stream(stream))


def swiglu_pack_down(Wdown, Wdpacked, d, dff, dtype, stream=None) -> int:
    return _lib.swiglu_pack_down(_ptr(Wdown), _ptr(Wdpacked), d, dff, dtype, _stream(stream))


def swiglu_up(x, Wpacked, out, M, d, dff, dtype, workspace=None, workspace_bytes=0,
              stream=None) -> int:
    return _lib.swiglu_up(_ptr(x), _ptr(Wpacked), _ptr(out), M, d, dff, dtype, _ptr(workspace),
                          workspace_bytes, _stream(stream))


def swiglu_up_ex(x, Wpacked, out, M, d, dff, dtype, workspace=None, workspace_bytes=0,
                 stream=None, path=SWIGLU_PATH_AUTO) -> int:
    return _lib.swiglu_up_ex(_ptr(x), _ptr(Wpacked), _ptr(out), M, d, dff, dtype,
                             _ptr(workspace), workspace_bytes, _stream(stream), path)


def swiglu_up_noalloc(x, Wpacked, out, M, d, dff, dtype, stream=None) -> int:
    return _lib.swiglu_up_noalloc(_ptr(x), _ptr(Wpacked), _ptr(out), M, d, dff, dtype,
                                  _stream(stream))


def mlp_forward(x, Wpacked, Wdpacked, y, M, d, dff, dtype, workspace=None, workspace_bytes=0,
                stream=None) -> int:
    return _lib.mlp_forward(_ptr(x), _ptr(Wpacked), _ptr(Wdpacked), _ptr(y), M, d, dff, dtype,
                            _ptr(workspace), workspace_bytes, _stream(stream))


def mlp_forward_ex(x, Wpacked, Wdpacked, y, M, d, dff, dtype, workspace=None, workspace_bytes=0,
                   stream=None, path=SWIGLU_PATH_AUTO) -> int:
    return _lib.mlp_forward_ex(_ptr(x), _ptr(Wpacked), _ptr(Wdpacked), _ptr(y), M, d, dff,
                               dtype, _ptr(workspace), workspace_bytes, _stream(stream), path)


def mlp_block_workspace_bytes(M, d, dff, dtype) -> int:
    return _lib.mlp_block_workspace_bytes(M, d, dff, dtype)


def mlp_block_workspace_bytes_ex(M, d, dff, dtype, path) -> int:
    return _lib.mlp_block_workspace_bytes_ex(M, d, dff, dtype, path)


def mlp_block_forward(r, gamma, eps, Wpacked, Wdpacked, bias, out, M, d, dff, dtype,
                      workspace=None, workspace_bytes=0, stream=None) -> int:
    return _lib.mlp_block_forward(_ptr(r), _ptr(gamma), eps, _ptr(Wpacked), _ptr(Wdpacked),
                                  _ptr(bias), _ptr(out), M, d, dff, dtype, _ptr(workspace),
                                  workspace_bytes, _stream(stream))


def mlp_block_forward_ex(r, gamma, eps, Wpacked, Wdpacked, bias, out, M, d, dff, dtype,
                         workspace=None, workspace_bytes=0, stream=None,
                         path=SWIGLU_PATH_AUTO) -> int:
    return _lib.mlp_block_forward_ex(_ptr(r), _ptr(gamma), eps, _ptr(Wpacked), _ptr(Wdpacked),
                                     _ptr(bias), _ptr(out), M, d, dff, dtype, _ptr(workspace),
                                     workspace_bytes, _stream(stream), path)


def swiglu_up_graph_create(x, Wpacked, out, M, d, dff, dtype, workspace=None, workspace_bytes=0,
                           path=SWIGLU_PATH_AUTO):
    """Returns (status, handle); the handle (an int) is None unless status is 0."""
    h = _vp()
    rc = _lib.swiglu_up_graph_create(_ptr(x), _ptr(Wpacked), _ptr(out), M, d, dff, dtype,
                                     _ptr(workspace), workspace_bytes, path, ctypes.byref(h))
    return rc, h.value


def mlp_forward_graph_create(x, Wpacked, Wdpacked, y, M, d, dff, dtype, workspace=None,
                             workspace_bytes=0, path=SWIGLU_PATH_AUTO):
    """Returns (status, handle); the handle (an int) is None unless status is 0."""
    h = _vp()
    rc = _lib.mlp_forward_graph_create(_ptr(x), _ptr(Wpacked), _ptr(Wdpacked), _ptr(y), M, d,
                                       dff, dtype, _ptr(workspace), workspace_bytes, path,
                                       ctypes.byref(h))
    return rc, h.value


def mlp_block_graph_create(r, gamma, eps, Wpacked, Wdpacked, bias, out, M, d, dff, dtype,
                           workspace=None, workspace_bytes=0, path=SWIGLU_PATH_AUTO):
    """Returns (status, handle); the handle (an int) is None unless status is 0."""
    h = _vp()
    rc = _lib.mlp_block_graph_create(_ptr(r), _ptr(gamma), eps, _ptr(Wpacked), _ptr(Wdpacked),
                                     _ptr(bias), _ptr(out), M, d, dff, dtype, _ptr(workspace),
                                     workspace_bytes, path, ctypes.byref(h))
    return rc, h.value


def swiglu_graph_launch(graph, stream=None) -> int:
    return _lib.swiglu_graph_launch(graph, _stream(stream))


def swiglu_graph_destroy(graph) -> int:
    return _lib.swiglu_graph_destroy(graph)


def check(status: int, what: str = "") -> None:
    """Raise SwigluError for a non-zero status."""
    if status != SWIGLU_OK:
        raise SwigluError(status, what)
