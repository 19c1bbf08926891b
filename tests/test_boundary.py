"""Host-only checks of the C-ABI library: it loads without a GPU, exports
every function include/swiglu.h declares, and rejects bad arguments before
any HIP call (so these run on a CPU-only machine)."""
import subprocess

import pytest

import gemv_gate_up_amd as sw
import workloads as wl

BF16, F32 = sw.SWIGLU_BF16, sw.SWIGLU_F32
FAKE = 0x10000000    # 16-byte aligned address that is never dereferenced here


def rejected_before_launch(create, direct, expected):
    """Checks a fake-pointer call whose rejection depends on the planner
    (the workspace it needs).  The graph-creation variant with the same
    arguments runs the same validation first, without any HIP call, and a
    recording never executes a kernel; only when it returns the expected
    status is the direct call made, so a planner change that made the call
    valid fails here instead of launching a kernel on a fake address."""
    rc, h = create()
    if h:
        sw.swiglu_graph_destroy(h)
    assert rc == expected, sw.swiglu_status_string(rc)
    assert direct() == expected


def test_header_symbols_are_exported():
    names = sw.header_functions()
    assert {"swiglu_pack_weights", "swiglu_up", "mlp_forward", "swiglu_pack_down"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", sw.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing


def test_status_strings_and_version():
    assert sw.swiglu_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert sw.swiglu_status_string(code) != "unknown status"
    assert sw.swiglu_status_string(17) == "unknown status"


def test_packed_sizes():
    # 8B-class: two 4096 x 14336 bf16 matrices, no padding needed
    assert sw.swiglu_packed_bytes(4096, 14336, BF16) == 2 * 4096 * 14336 * 2
    # 72B-class: dff = 29568 = 231 * 128 fits whole 256-column tiles
    assert sw.swiglu_packed_bytes(8192, 29568, BF16) == 968884224
    assert sw.swiglu_down_packed_bytes(8192, 29568, BF16) == 484442112
    # fp32 tiny decode
    assert sw.swiglu_packed_bytes(512, 2048, F32) == 2 * 512 * 2048 * 4
    # ragged shapes pad K to 64 (bf16) and columns to 128
    assert sw.swiglu_packed_bytes(1000, 1400, BF16) == 1024 * 1408 * 2 * 2
    assert sw.swiglu_packed_bytes(0, 16, BF16) == 0
    assert sw.swiglu_packed_bytes(16, 16, 7) == 0


def test_dispatcher():
    for M in (1, 4, 8, 16, 17, 32, 64):
        assert sw.swiglu_select_path(M, 4096, 14336, BF16) == sw.SWIGLU_PATH_SKINNY
    for M in (65, 128, 2048, 4096):
        assert sw.swiglu_select_path(M, 4096, 14336, BF16) == sw.SWIGLU_PATH_WIDE
    # above 64 rows the wide path needs enough workgroups: at least 128, or
    # 48 from 256 rows on.  The 0.5B-class gate/up product has 76 up to 256
    # rows and 152 at 512; the 72B-class shard (d_ff = 3696) 58 up to 256
    # rows; the 1.5B-class product (d_ff = 8960) 140 at 80 rows
    for M, d, dff, path in ((80, 896, 4864, 1), (128, 896, 4864, 1), (255, 896, 4864, 1),
                            (256, 896, 4864, 2), (512, 896, 4864, 2), (128, 8192, 3696, 1),
                            (256, 8192, 3696, 2), (80, 1536, 8960, 2)):
        assert sw.swiglu_select_path(M, d, dff, BF16) == path, (M, d, dff)
    for M in (1, 64, 4096):
        assert sw.swiglu_select_path(M, 512, 2048, F32) == sw.SWIGLU_PATH_SKINNY
    assert sw.swiglu_select_path(1, 4096, 14336, 9) == sw.SWIGLU_ERR_UNSUPPORTED
    assert sw.swiglu_select_path(-1, 4096, 14336, BF16) == sw.SWIGLU_ERR_INVALID_ARG


def test_workspace_sizes():
    # decode: the pair blocks fill the GPU, no split-K partials needed
    assert sw.swiglu_workspace_bytes(1, 4096, 14336, BF16, 0) == 0
    # the tiny fp32 decode streams 64 KB per pair block: not worth a split
    assert sw.swiglu_workspace_bytes(1, 512, 2048, F32, 0) == 0
    # a long K over 512 columns (32 pair blocks, 512 KB each) splits it 16
    # ways: 16 slices x 1 row x 1024 packed columns x 4 B of partials
    assert sw.swiglu_workspace_bytes(1, 4096, 512, F32, 0) == 16 * 1024 * 4
    # full MLP keeps h (M x padded dff) in the workspace
    assert sw.swiglu_workspace_bytes(2048, 8192, 29568, BF16, 1) >= 2048 * 29568 * 2
    assert sw.swiglu_workspace_bytes_ex(4096, 512, 2048, F32, 0, sw.SWIGLU_PATH_WIDE) == 0


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_argument_errors_return_before_any_launch(dtype):
    M, d, dff = 4, 64, 64
    up = lambda *a, **k: sw.swiglu_up(*a, stream=0, **k)
    assert up(FAKE, FAKE, FAKE, -1, d, dff, dtype) == sw.SWIGLU_ERR_INVALID_ARG
    assert up(FAKE, FAKE, FAKE, M, 0, dff, dtype) == sw.SWIGLU_ERR_INVALID_ARG
    assert up(FAKE, FAKE, FAKE, M, d, -8, dtype) == sw.SWIGLU_ERR_INVALID_ARG
    assert up(FAKE, FAKE, FAKE, M, d, dff, 5) == sw.SWIGLU_ERR_UNSUPPORTED
    assert up(FAKE, FAKE, FAKE, M, 6, dff, dtype) == sw.SWIGLU_ERR_UNSUPPORTED
    assert up(FAKE, FAKE, FAKE, M, d, (1 << 20) + 8, dtype) == sw.SWIGLU_ERR_UNSUPPORTED
    assert up(None, FAKE, FAKE, M, d, dff, dtype) == sw.SWIGLU_ERR_INVALID_ARG
    assert up(FAKE, None, FAKE, M, d, dff, dtype) == sw.SWIGLU_ERR_INVALID_ARG
    assert up(FAKE + 4, FAKE, FAKE, M, d, dff, dtype) == sw.SWIGLU_ERR_MISALIGNED
    assert up(FAKE, FAKE, FAKE + 8, M, d, dff, dtype) == sw.SWIGLU_ERR_MISALIGNED
    # M == 0 is a no-op, whatever the pointers
    assert up(None, None, None, 0, d, dff, dtype) == sw.SWIGLU_OK
    assert sw.mlp_forward(None, None, None, None, 0, d, dff, dtype, stream=0) == sw.SWIGLU_OK
    assert sw.mlp_forward(FAKE, FAKE, FAKE, FAKE, M, d, dff, dtype, None, 0,
                          stream=0) == sw.SWIGLU_ERR_INVALID_ARG
    assert sw.swiglu_pack_weights(FAKE, None, FAKE, d, dff, dtype, 0) == sw.SWIGLU_ERR_INVALID_ARG
    assert sw.swiglu_pack_weights(FAKE, FAKE + 2, FAKE, d, dff, dtype, 0) == sw.SWIGLU_ERR_MISALIGNED
    assert sw.swiglu_pack_down(FAKE, FAKE, d, 0, dtype, 0) == sw.SWIGLU_ERR_INVALID_ARG


def test_workspace_too_small_is_rejected():
    # a split-K decode needs partials; none are given
    assert sw.swiglu_workspace_bytes(1, 4096, 512, F32, 0) > 0
    rejected_before_launch(
        lambda: sw.swiglu_up_graph_create(FAKE, FAKE, FAKE, 1, 4096, 512, F32, None, 0),
        lambda: sw.swiglu_up(FAKE, FAKE, FAKE, 1, 4096, 512, F32, None, 0, stream=0),
        sw.SWIGLU_ERR_WORKSPACE)
    need = sw.swiglu_workspace_bytes(64, 896, 4864, BF16, 1)
    rejected_before_launch(
        lambda: sw.mlp_forward_graph_create(FAKE, FAKE, FAKE, FAKE, 64, 896, 4864, BF16, FAKE,
                                            need - 256),
        lambda: sw.mlp_forward(FAKE, FAKE, FAKE, FAKE, 64, 896, 4864, BF16, FAKE, need - 256,
                               stream=0),
        sw.SWIGLU_ERR_WORKSPACE)


def test_forced_paths():
    rc = sw.swiglu_up_ex(FAKE, FAKE, FAKE, 4, 64, 64, F32, None, 0, 0, sw.SWIGLU_PATH_WIDE)
    assert rc == sw.SWIGLU_ERR_UNSUPPORTED
    rc = sw.swiglu_up_ex(FAKE, FAKE, FAKE, 4, 64, 64, F32, None, 0, 0,
                         sw.SWIGLU_PATH_WIDE_PHASED)
    assert rc == sw.SWIGLU_ERR_UNSUPPORTED
    rc = sw.swiglu_up_ex(FAKE, FAKE, FAKE, 4, 64, 64, BF16, None, 0, 0, 4)
    assert rc == sw.SWIGLU_ERR_UNSUPPORTED
    # both many-rows schedules take x packed into the workspace: one 1 KB
    # piece per 16 rows x 32 K (they also run without it, on x in place)
    packed_x = (4096 // 16) * (4096 // 32) * 1024
    for path in (sw.SWIGLU_PATH_WIDE, sw.SWIGLU_PATH_WIDE_PHASED, sw.SWIGLU_PATH_AUTO):
        assert sw.swiglu_workspace_bytes_ex(4096, 4096, 14336, BF16, 0, path) == packed_x
    # rows padded to 16, K to the weight's 64
    assert sw.swiglu_workspace_bytes_ex(130, 264, 712, BF16, 0, sw.SWIGLU_PATH_WIDE) == \
        9 * 10 * 1024
    assert sw.swiglu_workspace_bytes_ex(96, 512, 1408, BF16, 1, sw.SWIGLU_PATH_WIDE_PHASED) == \
        sw.swiglu_workspace_bytes_ex(96, 512, 1408, BF16, 1, sw.SWIGLU_PATH_WIDE)


def test_workloads_shapes_are_supported():
    for w in wl.WORKLOADS.values():
        assert sw.swiglu_packed_bytes(w.d, w.dff, w.dtype) > 0
        assert sw.swiglu_select_path(w.M, w.d, w.dff, w.dtype) in (1, 2)


def test_graph_create_rejects_bad_arguments_before_any_hip_call():
    # the same checks as the direct calls, made before a stream is created
    rc, h = sw.swiglu_up_graph_create(FAKE, FAKE, FAKE, -1, 64, 64, BF16)
    assert (rc, h) == (sw.SWIGLU_ERR_INVALID_ARG, None)
    rc, h = sw.swiglu_up_graph_create(FAKE + 4, FAKE, FAKE, 4, 64, 64, BF16)
    assert (rc, h) == (sw.SWIGLU_ERR_MISALIGNED, None)
    rc, h = sw.swiglu_up_graph_create(FAKE, FAKE, FAKE, 1, 4096, 512, F32, None, 0)
    assert (rc, h) == (sw.SWIGLU_ERR_WORKSPACE, None)
    rc, h = sw.swiglu_up_graph_create(FAKE, FAKE, FAKE, 4, 64, 64, F32, None, 0,
                                      sw.SWIGLU_PATH_WIDE)
    assert (rc, h) == (sw.SWIGLU_ERR_UNSUPPORTED, None)
    rc, h = sw.mlp_forward_graph_create(FAKE, FAKE, FAKE, FAKE, 4, 64, 64, BF16, None, 0)
    assert (rc, h) == (sw.SWIGLU_ERR_INVALID_ARG, None)
    assert sw._lib.swiglu_up_graph_create(FAKE, FAKE, FAKE, 4, 64, 64, BF16, None, 0, 0,
                                          None) == sw.SWIGLU_ERR_INVALID_ARG
    rc, h = sw.mlp_block_graph_create(FAKE, FAKE, -1.0, FAKE, FAKE, None, FAKE, 4, 64, 64, BF16,
                                      FAKE, 1 << 20)
    assert (rc, h) == (sw.SWIGLU_ERR_INVALID_ARG, None)
    assert sw.swiglu_graph_launch(None, 0) == sw.SWIGLU_ERR_INVALID_ARG
    assert sw.swiglu_graph_destroy(None) == sw.SWIGLU_OK


def test_one_hip_runtime_in_the_process():
    # importing the binding must not map a second libamdhip64 beside torch's
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read().split("\n")
    files = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(files) == 1, files


def test_fp8_weight_sizes_and_paths():
    W8 = sw.SWIGLU_BF16_FP8W
    # one byte per weight, K padded to 64, then one fp32 scale per packed column
    assert sw.swiglu_packed_bytes(4096, 14336, W8) == 4096 * 14336 * 2 + 896 * 32 * 4
    # K 104 -> 128; 40 columns -> 3 pair blocks -> 8 (128 packed columns per half)
    assert sw.swiglu_packed_bytes(104, 40, W8) == 128 * 128 * 2 + 8 * 32 * 4
    assert sw.swiglu_packed_bytes(100, 40, W8) == 0
    assert sw.swiglu_down_packed_bytes(8192, 29568, W8) == 29568 * 8192 + 256 * 32 * 4
    for M in (1, 64, 65, 4096):
        assert sw.swiglu_select_path(M, 4096, 14336, W8) == sw.SWIGLU_PATH_SKINNY
    for path in (sw.SWIGLU_PATH_WIDE, sw.SWIGLU_PATH_WIDE_PHASED):
        rc = sw.swiglu_up_ex(FAKE, FAKE, FAKE, 4, 64, 64, W8, None, 0, 0, path)
        assert rc == sw.SWIGLU_ERR_UNSUPPORTED
    # activations stay bf16: d and dff multiples of 8
    assert sw.swiglu_up(FAKE, FAKE, FAKE, 1, 68, 64, W8, None, 0, stream=0) == \
        sw.SWIGLU_ERR_UNSUPPORTED
    # the down product's h is bf16 in the workspace, like the bf16 dtype
    assert sw.swiglu_workspace_bytes(16, 8192, 29568, W8, 1) >= 16 * 29568 * 2


def test_mlp_block_arguments_and_workspace():
    M, d, dff = 4, 64, 64
    need = sw.mlp_block_workspace_bytes(M, d, dff, BF16)
    # the normalised rows come first, then the MLP's own workspace
    assert need == 256 * -(-(M * d * 2) // 256) + sw.swiglu_workspace_bytes(M, d, dff, BF16, 1)
    # on the many-rows path RMSNorm writes its rows already packed, in the
    # place the MLP would pack x into
    assert sw.mlp_block_workspace_bytes(4096, 4096, 14336, BF16) == \
        sw.swiglu_workspace_bytes(4096, 4096, 14336, BF16, 1)
    blk = lambda *a, **k: sw.mlp_block_forward(*a, stream=0, **k)
    assert blk(FAKE, FAKE, 1e-5, FAKE, FAKE, None, FAKE, 0, d, dff, BF16) == sw.SWIGLU_OK
    assert blk(FAKE, FAKE, -1.0, FAKE, FAKE, None, FAKE, M, d, dff, BF16, FAKE,
               need) == sw.SWIGLU_ERR_INVALID_ARG
    assert blk(FAKE, FAKE, float("nan"), FAKE, FAKE, None, FAKE, M, d, dff, BF16, FAKE,
               need) == sw.SWIGLU_ERR_INVALID_ARG
    assert blk(FAKE, None, 1e-5, FAKE, FAKE, None, FAKE, M, d, dff, BF16, FAKE,
               need) == sw.SWIGLU_ERR_INVALID_ARG
    assert blk(FAKE, FAKE, 1e-5, FAKE, FAKE, FAKE + 1, FAKE, M, d, dff, BF16, FAKE,
               need) == sw.SWIGLU_ERR_MISALIGNED
    rejected_before_launch(
        lambda: sw.mlp_block_graph_create(FAKE, FAKE, 1e-5, FAKE, FAKE, None, FAKE, M, d, dff,
                                          BF16, FAKE, need - 256),
        lambda: blk(FAKE, FAKE, 1e-5, FAKE, FAKE, None, FAKE, M, d, dff, BF16, FAKE, need - 256),
        sw.SWIGLU_ERR_WORKSPACE)
    assert sw.mlp_block_forward_ex(FAKE, FAKE, 1e-5, FAKE, FAKE, None, FAKE, M, d, dff, F32, FAKE,
                                   need, 0, sw.SWIGLU_PATH_WIDE) == sw.SWIGLU_ERR_UNSUPPORTED


def test_mxfp4_weight_sizes_and_paths():
    W4 = sw.SWIGLU_BF16_MXFP4W
    # half a byte per weight (K padded to 128), one scale byte per 32 weights
    assert sw.swiglu_packed_bytes(4096, 14336, W4) == 4096 * 14336 + 4096 * 14336 * 2 // 32
    assert sw.swiglu_packed_bytes(136, 40, W4) == 256 * 128 + 256 * 128 * 2 // 32
    for M in (1, 64, 65):
        assert sw.swiglu_select_path(M, 4096, 14336, W4) == sw.SWIGLU_PATH_SKINNY
    rc = sw.swiglu_up_ex(FAKE, FAKE, FAKE, 4, 64, 64, W4, None, 0, 0, sw.SWIGLU_PATH_WIDE)
    assert rc == sw.SWIGLU_ERR_UNSUPPORTED


def test_header_is_plain_c_and_links(tmp_path):
    # a C99 program against include/swiglu.h, linked with libswiglu.so; it
    # exercises argument checks only, so it runs without a GPU
    import os
    src = os.path.join(os.path.dirname(__file__), "c", "abi_check.c")
    exe = str(tmp_path / "abi_check")
    libdir = os.path.dirname(sw.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.dirname(sw.HEADER_PATH), "-I", "/opt/rocm/include", src, "-o", exe,
           "-L", libdir, "-lswiglu", "-Wl,-rpath," + libdir]
    subprocess.run(["ln", "-sf", sw.LIB_PATH, str(tmp_path / "libswiglu.so")], check=True)
    cmd[cmd.index("-L") + 1] = str(tmp_path)
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # every GPU hidden from the program (HIP reports no device), so a call
    # that wrongly passed validation could not launch on a placeholder address
    env = dict(os.environ, ROCR_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check ok" in r.stdout


def _packed_bytes(M, K):
    """Packed activations: one 1 KB piece per 16 rows x 32 K, K padded to 64."""
    return -(-M // 16) * (-(-K // 64) * 2) * 1024


def _al(n):
    return -(-n // 256) * 256


# the last shape is ragged in M, d and dff, with both products still on the
# wide path (108 and 50 workgroups at 300 rows)
@pytest.mark.parametrize("shape", [(4096, 4096, 14336), (2048, 8192, 29568), (300, 3080, 3400)])
def test_packed_plan_workspace_formulas(shape):
    M, d, dff = shape
    assert sw.swiglu_select_path(M, d, dff, BF16) == sw.SWIGLU_PATH_WIDE
    # swiglu_up on the many-rows path: packed x only
    assert sw.swiglu_workspace_bytes(M, d, dff, BF16, 0) == _al(_packed_bytes(M, d))
    # mlp_forward: h packed for the down product, then packed x (no split-K partials)
    assert sw.swiglu_workspace_bytes(M, d, dff, BF16, 1) == \
        _al(_packed_bytes(M, dff)) + _al(_packed_bytes(M, d))
    # the block: RMSNorm's packed rows take the place of packed x
    assert sw.mlp_block_workspace_bytes(M, d, dff, BF16) == \
        sw.swiglu_workspace_bytes(M, d, dff, BF16, 1)


def test_workspace_below_the_row_major_plan_is_rejected():
    # the row-major plan of mlp_forward keeps h as M x padded-dff bf16; one
    # allocation unit less than that fails before any launch
    M, d, dff = 300, 3080, 3400   # both products on the wide path
    row_major = _al(M * (-(-dff // 128) * 128) * 2)
    assert sw.swiglu_workspace_bytes(M, d, dff, BF16, 1) > row_major
    rejected_before_launch(
        lambda: sw.mlp_forward_graph_create(FAKE, FAKE, FAKE, FAKE, M, d, dff, BF16, FAKE,
                                            row_major - 256),
        lambda: sw.mlp_forward(FAKE, FAKE, FAKE, FAKE, M, d, dff, BF16, FAKE, row_major - 256,
                               stream=0),
        sw.SWIGLU_ERR_WORKSPACE)
    blk_bytes = _al(M * d * 2) + row_major - 256
    rejected_before_launch(
        lambda: sw.mlp_block_graph_create(FAKE, FAKE, 1e-6, FAKE, FAKE, None, FAKE, M, d, dff,
                                          BF16, FAKE, blk_bytes),
        lambda: sw.mlp_block_forward(FAKE, FAKE, 1e-6, FAKE, FAKE, None, FAKE, M, d, dff, BF16,
                                     FAKE, blk_bytes, stream=0),
        sw.SWIGLU_ERR_WORKSPACE)


def test_noalloc_rejects_bad_arguments_before_any_hip_call():
    # the entry point without a workspace checks its arguments and its plan
    # (which must fit the library's fixed array) before looking up the
    # array's device address or launching anything
    up = sw.swiglu_up_noalloc
    assert up(FAKE, FAKE, FAKE, -1, 64, 64, BF16, stream=0) == sw.SWIGLU_ERR_INVALID_ARG
    assert up(None, FAKE, FAKE, 4, 64, 64, BF16, stream=0) == sw.SWIGLU_ERR_INVALID_ARG
    assert up(FAKE, FAKE, FAKE, 4, 64, 64, 7, stream=0) == sw.SWIGLU_ERR_UNSUPPORTED
    assert up(FAKE, FAKE, FAKE, 4, 68, 64, BF16, stream=0) == sw.SWIGLU_ERR_UNSUPPORTED
    assert up(FAKE + 4, FAKE, FAKE, 4, 64, 64, BF16, stream=0) == sw.SWIGLU_ERR_MISALIGNED
    assert up(None, None, None, 0, 64, 64, BF16, stream=0) == sw.SWIGLU_OK
    assert sw.swiglu_status_string(sw.SWIGLU_ERR_SCRATCH) != "unknown status"


def test_noalloc_scratch_covers_every_plan():
    # the array holds any shape's split-K partials (the largest, on the
    # forced few-rows path, is 16 MiB) and the 8B-class prefill's packed x;
    # larger packed x falls back to reading x in place
    assert sw.swiglu_workspace_bytes_ex(256, 32768, 8, BF16, 0, sw.SWIGLU_PATH_SKINNY) <= \
        sw.SWIGLU_SCRATCH_BYTES
    assert sw.swiglu_workspace_bytes(4096, 4096, 14336, BF16, 0) == sw.SWIGLU_SCRATCH_BYTES
    assert sw.swiglu_workspace_bytes(4608, 4096, 512, BF16, 0) > sw.SWIGLU_SCRATCH_BYTES
    assert sw.swiglu_workspace_bytes_ex(4608, 4096, 512, BF16, 0, sw.SWIGLU_PATH_SKINNY) == 0


def test_fused_down_path_sizes_and_rejections():
    F = sw.SWIGLU_PATH_FUSED_DOWN
    # the fused MLP's workspace holds one fp32 slice of y (d padded to 256
    # columns) per d_ff slice: four 16-column pair blocks per slice at 64 rows
    slices = -(-4864 // 16) // 4
    assert sw.swiglu_workspace_bytes_ex(64, 896, 4864, BF16, 1, F) == \
        _al(slices * 64 * 1024 * 4)
    # eight pair blocks per slice at up to 16 rows
    assert sw.swiglu_workspace_bytes_ex(16, 8192, 29568, BF16, 1, F) == \
        _al(-(-(29568 // 16) // 8) * 16 * 8192 * 4)
    # bf16 MLPs only: swiglu_up, fp32 and quantised weights are rejected
    # before any launch
    assert sw.swiglu_workspace_bytes_ex(64, 896, 4864, BF16, 0, F) == 0
    assert sw.swiglu_up_ex(FAKE, FAKE, FAKE, 4, 64, 64, BF16, None, 0, 0, F) == \
        sw.SWIGLU_ERR_UNSUPPORTED
    for dt in (F32, sw.SWIGLU_BF16_FP8W, sw.SWIGLU_BF16_MXFP4W):
        assert sw.mlp_forward_ex(FAKE, FAKE, FAKE, FAKE, 4, 64, 64, dt, FAKE, 1 << 20, 0, F) == \
            sw.SWIGLU_ERR_UNSUPPORTED
    need = sw.swiglu_workspace_bytes_ex(64, 896, 4864, BF16, 1, F)
    rejected_before_launch(
        lambda: sw.mlp_forward_graph_create(FAKE, FAKE, FAKE, FAKE, 64, 896, 4864, BF16, FAKE,
                                            need - 256, F),
        lambda: sw.mlp_forward_ex(FAKE, FAKE, FAKE, FAKE, 64, 896, 4864, BF16, FAKE, need - 256,
                                  0, F),
        sw.SWIGLU_ERR_WORKSPACE)
