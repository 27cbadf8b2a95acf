"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU code (no GPU).

* The oracle: oracle.c built with gcc's sanitizers, then every entry point
  driven on small and edge-case inputs (tests/sanitizer_oracle_calls.py) in a
  process that preloads gcc's ASan runtime.  A control build with a planted
  one-past-the-end write must be caught, so a sanitizer that silently does not
  run cannot pass the test.
* The library's host code: api.hip (argument validation, workspace sizing)
  compiled with the sanitizers on its host side only (each -fsanitize= behind
  -Xarch_host; device code is unchanged) and linked with the other objects,
  then tests/test_abi.py run against it in a process that preloads clang's
  ASan runtime.  Every call there fails validation or is an empty problem, so
  no HIP call is made.  A control library with a planted out-of-bounds host
  read, built the same way, must be caught.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
DRIVER = os.path.join(ROOT, "tests", "sanitizer_oracle_calls.py")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "2"}


def _gcc_asan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _clang_asan():
    from compressed_latent_causal_amd import build as B
    clang = os.path.join(os.path.dirname(os.path.realpath(B.hipcc())), "..", "lib", "llvm", "bin",
                         "clang")
    cands = []
    if os.path.exists(clang):
        p = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                           capture_output=True, text=True).stdout.strip()
        cands.append(p)
    cands += glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    for p in cands:
        if os.path.isabs(p) and os.path.exists(p):
            return p
    pytest.skip("clang's AddressSanitizer runtime is not installed")


def _gcc_san_build(src, out):
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-shared", "-fPIC", "-Wall", src, "-o", out, "-lm"],
                   check=True)


def _run(cmd, runtime, extra_env, timeout=600):
    env = dict(os.environ, LD_PRELOAD=runtime, **SAN_ENV, **extra_env)
    return subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_oracle_under_asan_and_ubsan(tmp_path):
    asan = _gcc_asan()
    lib = str(tmp_path / "liboracle_san.so")
    _gcc_san_build(ORACLE_SRC, lib)
    r = _run([sys.executable, DRIVER], asan, {"ORACLE_LIB": lib})
    assert r.returncode == 0 and "all oracle calls done" in r.stdout, r.stderr[-4000:]


def test_oracle_sanitizer_catches_a_planted_overflow(tmp_path):
    asan = _gcc_asan()
    text = open(ORACLE_SRC).read()
    old = "for (size_t i = 0; i < n; ++i)\n        out[i] = round_bf16(in[i]);"
    assert text.count(old) == 1
    src = tmp_path / "oracle_overflow.c"
    src.write_text(text.replace(old, old.replace("i < n", "i <= n")))
    lib = str(tmp_path / "liboracle_overflow.so")
    _gcc_san_build(str(src), lib)
    r = _run([sys.executable, DRIVER], asan, {"ORACLE_LIB": lib})
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.returncode, r.stderr[-2000:])


HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _host_san_lib(tmp_path, api_src):
    """libattn with api_src's host code sanitized; the kernels' objects as the
    in-tree build makes them (reused when newer than every source)."""
    from compressed_latent_causal_amd import build as B
    bdir = str(tmp_path / "objs")
    os.makedirs(bdir, exist_ok=True)
    headers = [os.path.join(B.CSRC, h) for h in ("common.hpp", "kernels.hpp")] + [
        os.path.join(ROOT, "include", "attn.h")]

    def obj(src):
        built = os.path.join(B.BUILD, os.path.splitext(src)[0] + ".o")
        newest = max(os.path.getmtime(p) for p in headers + [os.path.join(B.CSRC, src)])
        if os.path.exists(built) and os.path.getmtime(built) > newest:
            return built
        return B._compile(src, bdir)

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(obj, [s for s in B.SOURCES if s != "api.hip"]))
    api_obj = os.path.join(bdir, "api_san.o")
    subprocess.run([B.hipcc(), *B.COMMON_FLAGS, "-g", *HOST_SAN, "-c", api_src, "-o", api_obj],
                   check=True, capture_output=True, text=True)
    out = str(tmp_path / "libattn_san.so")
    subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", out, api_obj,
                    *objs], check=True, capture_output=True, text=True)
    return out


_ABI_RUNNER = """
import sys
from compressed_latent_causal_amd import _lib
_lib.lib_path = lambda: sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "tests/test_abi.py",
                      "-k", "not fails_loudly"]))
"""


def test_host_validation_under_asan_and_ubsan(tmp_path):
    asan = _clang_asan()
    from compressed_latent_causal_amd import build as B
    lib = _host_san_lib(tmp_path, os.path.join(B.CSRC, "api.hip"))
    r = _run([sys.executable, "-c", _ABI_RUNNER, lib], asan, {})
    assert r.returncode == 0 and " passed" in r.stdout, (r.stdout[-3000:], r.stderr[-3000:])


def test_host_sanitizer_catches_a_planted_overread(tmp_path):
    """The same build and runtime catch a host read past a heap block: a
    control library whose attn_status_string reads one entry past a malloc'd
    array (the planted fault lives in a copy of api.hip under tmp_path)."""
    asan = _clang_asan()
    from compressed_latent_causal_amd import build as B
    text = open(os.path.join(B.CSRC, "api.hip")).read()
    marker = "ATTN_API const char* attn_status_string(int status) {"
    assert text.count(marker) == 1, "attn_status_string definition not found"
    planted = marker + (
        "\n    if (status == 12345) {\n"
        "        int* probe = (int*)malloc(4 * sizeof(int));\n"
        "        volatile int idx = 4;\n"
        "        const int x = probe[idx];\n"
        "        free(probe);\n"
        "        return x ? \"x\" : \"y\";\n"
        "    }\n")
    src = tmp_path / "api.hip"
    src.write_text("#include <stdlib.h>\n" + text.replace(marker, planted).replace(
        '#include "../../include/attn.h"', f'#include "{ROOT}/include/attn.h"'))
    for h in ("common.hpp", "kernels.hpp"):
        (tmp_path / h).write_text(open(os.path.join(B.CSRC, h)).read())
    lib = _host_san_lib(tmp_path, str(src))
    code = ("import ctypes, sys\nL = ctypes.CDLL(sys.argv[1])\n"
            "L.attn_status_string.restype = ctypes.c_char_p\n"
            "L.attn_status_string(12345)\nprint('not caught')\n")
    r = _run([sys.executable, "-c", code, lib], asan, {})
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.returncode, r.stderr[-2000:])
