"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only, no GPU): the oracle built with gcc -fsanitize=address,undefined runs
every pin, and the C ABI layer (pkm_api.hip, host side instrumented, linked
with the library's other objects as built) runs every argument-check test of
test_abi.py.  Each run is a child process with the sanitizer runtime
preloaded; any report aborts it (no recovery), which fails the test."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, env_extra, timeout=900):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=timeout, cwd=ROOT)
    assert res.returncode == 0, (res.stdout[-3000:] + res.stderr[-3000:])
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr
    return res


def test_oracle_pins_under_asan_ubsan():
    import oracle
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.exists(libasan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.build(out=os.path.join(d, "liborc_san.so"),
                           extra_flags=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                        "-fno-omit-frame-pointer", "-g"))
        script = ("import sys; sys.path[:0] = [%r, %r]\n"
                  "import oracle, oracle_pins\n"
                  "bad = oracle_pins.failing_pins(oracle.Oracle(%r))\n"
                  "assert not bad, bad\n"
                  "print('pins ok', len(oracle_pins.ALL_PINS))\n") % (ROOT, TESTS, lib)
        res = _run([sys.executable, "-c", script], {"LD_PRELOAD": libasan, "OMP_NUM_THREADS": "4"})
        assert "pins ok" in res.stdout


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_layer_under_asan_ubsan():
    from product_key_memory_amd import build as B
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("the ROCm clang AddressSanitizer runtime is not installed")
    B.build_library(incremental=True)          # the other objects, as built (reused when current)
    objs = [o for o in glob.glob(os.path.join(B.OBJ_DIR, "*.o"))
            if not os.path.basename(o).startswith("pkm_api.hip")]
    with tempfile.TemporaryDirectory() as d:
        api_o = os.path.join(d, "api_san.o")
        host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                    "-fno-omit-frame-pointer"]
        flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
        subprocess.run([B.hipcc(), *flags, *host_san, "-I", B.INCLUDE, "-I", B.CSRC, "-c",
                        os.path.join(B.CSRC, "pkm_api.hip"), "-o", api_o],
                       check=True, capture_output=True)
        lib = os.path.join(d, "libpkm_san.so")
        subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-shared-libsan", api_o, *objs, "-o", lib], check=True, capture_output=True)
        nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in nm, "the ABI layer is not instrumented"
        res = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                    os.path.join(TESTS, "test_abi.py")],
                   {"LD_PRELOAD": rt, "PKM_LIB": lib, "LD_LIBRARY_PATH": os.path.dirname(rt)})
        assert " passed" in res.stdout
