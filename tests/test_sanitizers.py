"""AddressSanitizer / UndefinedBehaviorSanitizer runs of the host code (CPU only).

* The CPU oracle (``oracle/oracle.c``, gcc) under a C driver that computes
  every oracle function on small ragged inputs and feeds each one inputs it
  must reject (``tests/sanitize_oracle.c``).
* The library's host side (``api.hip`` compiled with host-only instrumentation,
  linked with the uninstrumented kernel objects of the normal build) under a C
  driver that calls every entry point with arguments it must reject before any
  HIP call, and sweeps the size queries (``tests/sanitize_api.c``).
* The CPU test suite itself, in a child Python with the clang ASan runtime
  preloaded, loading both instrumented libraries (``BTK_ORACLE_LIB``,
  ``BTK_LIB``).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "block_top_sparse_btk_amd", "csrc")
OBJS = os.path.join(ROOT, "block_top_sparse_btk_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
# every object of the normal build except the C ABI's own
from block_top_sparse_btk_amd import build as _hip_build  # noqa: E402

KERNEL_OBJS = [s.replace(".hip", ".o") for s in _hip_build.SOURCES if s != "api.hip"]


def _host_only(flags):
    """Each flag applies to the host compilation only (device code is not instrumented)."""
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n--- stdout\n{r.stdout[-4000:]}\n--- stderr\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def sanbuild(tmp_path_factory):
    for tool in ("gcc", HIPCC, CLANG):
        if not shutil.which(tool):
            pytest.skip(f"{tool} not available")
    d = tmp_path_factory.mktemp("sanitize")
    out = {}
    # oracle driver (gcc's runtime)
    out["oracle_driver"] = str(d / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", *SAN, "-o", out["oracle_driver"],
          os.path.join(TESTS, "sanitize_oracle.c"), os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    # oracle library for the preloaded suite run (clang's runtime, like the HIP host code)
    out["oracle_lib"] = str(d / "liboracle_san.so")
    _run([CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", *SAN, "-o", out["oracle_lib"],
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    # library: api.hip instrumented on the host side, kernels from the normal build
    if not all(os.path.exists(os.path.join(OBJS, o)) for o in KERNEL_OBJS):
        from block_top_sparse_btk_amd import build as hip_build
        hip_build.build()
    api_o = str(d / "api.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-I",
          os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", *_host_only(SAN), "-c", os.path.join(CSRC, "api.hip"), "-o", api_o])
    out["lib"] = str(d / "libbtk_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out["lib"], api_o,
          *[os.path.join(OBJS, o) for o in KERNEL_OBJS]])
    out["api_driver"] = str(d / "api_driver")
    _run([CLANG, "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"), "-o", out["api_driver"],
          os.path.join(TESTS, "sanitize_api.c"), out["lib"], f"-Wl,-rpath,{d}", "-lm"])
    out["asan_rt"] = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                    capture_output=True, text=True, check=True).stdout.strip()
    return out


def _env(**extra):
    env = dict(os.environ)
    env.update(extra)
    return env


def test_oracle_under_asan_ubsan(sanbuild):
    r = _run([sanbuild["oracle_driver"]], env=_env(ASAN_OPTIONS="detect_leaks=1",
                                                   OMP_NUM_THREADS="4"))
    assert "ok" in r.stdout


def test_api_validation_under_asan_ubsan(sanbuild):
    r = _run([sanbuild["api_driver"]], env=_env(ASAN_OPTIONS="detect_leaks=1"))
    assert "ok" in r.stdout


@pytest.mark.skipif(os.environ.get("BTK_LIB") is not None, reason="already the instrumented run")
def test_cpu_suite_under_asan(sanbuild):
    """The CPU tests of the oracle and the C ABI, with both instrumented libraries."""
    assert os.path.exists(sanbuild["asan_rt"]), sanbuild["asan_rt"]
    env = _env(LD_PRELOAD=sanbuild["asan_rt"], ASAN_OPTIONS="detect_leaks=0",
               BTK_ORACLE_LIB=sanbuild["oracle_lib"], BTK_LIB=sanbuild["lib"])
    files = [os.path.join(TESTS, f) for f in ("test_oracle_pins.py", "test_oracle_mutants.py",
                                               "test_parity_rules.py", "test_abi_cpu.py")]
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *files, "-k", "not sanitizer"]
    r = _run(cmd, env=env, timeout=1500)
    assert " passed" in r.stdout
    # both instrumented libraries were the ones loaded
    probe = ("import sys, oracle, block_top_sparse_btk_amd as b; oracle.lib(); b._lib(); "
             "m = open('/proc/self/maps').read(); "
             f"sys.exit(0 if {sanbuild['lib']!r} in m and {sanbuild['oracle_lib']!r} in m else 3)")
    _run([sys.executable, "-c", probe], env=env)
