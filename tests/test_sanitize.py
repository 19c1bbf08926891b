"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, with any
report fatal: the oracle (gcc), and the library's host side -- argument
checks, planners and size queries -- built by hipcc with the sanitizers on
the host pass only (the device code is built as usual and never run here).
Each is driven by a C program under tests/c that needs no GPU."""
import concurrent.futures
import os
import subprocess


HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
# every GPU hidden from the drivers (HIP then reports no device): their calls
# are all rejected before any launch, and if a change ever let one through
# it fails on the host instead of reaching a GPU with a placeholder address
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1",
           ROCR_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")


def _run(exe, marker):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert marker in r.stdout


def test_oracle_is_clean_under_sanitizers(tmp_path):
    # every oracle entry point: all bf16/E4M3/E2M1 patterns, non-finite
    # values, K not a multiple of 32, row subsets, optional outputs, one and
    # two threads
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-Wall", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(HERE, "c", "oracle_sanitize.c"), "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    _run(exe, "oracle_sanitize ok")


def test_library_host_code_is_clean_under_sanitizers(tmp_path):
    # the library's sources with its own flags, -O1, sanitizers on the host
    # pass; linked into a library the C driver loads
    from gemv_gate_up_amd import build as b
    flags = [f for f in b.CFLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        r = subprocess.run([b.HIPCC] + flags + san + ["-c", os.path.join(b.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, len(b.SOURCES))) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    lib = str(tmp_path / "libswiglu.so")
    r = subprocess.run([b.HIPCC, "--offload-arch=" + b.ARCH, "-shared", "-fPIC"] + san +
                       ["-o", lib] + objs, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "abi_sanitize")
    clang = os.path.join(os.path.dirname(os.path.realpath(b.HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-std=c99", "-Wall", "-Wextra", "-Werror", "-O1", "-g",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-D__HIP_PLATFORM_AMD__", "-I", b.INCLUDE, "-I", "/opt/rocm/include",
                        os.path.join(HERE, "c", "abi_sanitize.c"), "-o", exe,
                        "-L", str(tmp_path), "-lswiglu", "-Wl,-rpath," + str(tmp_path)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    _run(exe, "abi_sanitize ok")
