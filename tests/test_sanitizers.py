"""Host-side memory and undefined-behaviour checks (no GPU).

Builds, with gcc/g++ and -fsanitize=address,undefined (host code only):
  * the fp64 oracle (oracle/gda_ref.c), and
  * the C-ABI host layer (gda_api.cpp: argument validation, head grouping,
    dispatch), linked with the library's already-built kernel objects,
then runs the oracle pin tests and the C-ABI tests against those builds in a child
process with the sanitizer runtimes preloaded, so that any out-of-bounds access,
use after free, signed overflow or misaligned access on those paths aborts the run.
A planted heap overflow in a throwaway C file checks that the harness does abort.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "attention_gda_fwd_amd", "_build")
KERNEL_OBJS = ["gda_fwd_bf16.o", "gda_decode_bf16.o", "gda_f32.o", "gda_latent_bf16.o",
               "gda_bwd_bf16.o"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not found")
    return path


def _env(extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.fixture(scope="module")
def san_builds(tmp_path_factory):
    missing = [o for o in KERNEL_OBJS if not os.path.exists(os.path.join(BUILD, o))]
    if missing:
        pytest.skip(f"kernel objects not built ({missing}); run the library build first")
    d = tmp_path_factory.mktemp("san")
    oracle_so = str(d / "libgda_ref_san.so")
    _run(["gcc", *SAN, "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
          "-o", oracle_so, os.path.join(ROOT, "oracle", "gda_ref.c"), "-lm"])
    api_o = str(d / "gda_api.o")
    _run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"), "-fPIC", "-c",
          os.path.join(ROOT, "attention_gda_fwd_amd", "csrc", "gda_api.cpp"), "-o", api_o])
    lib_so = str(d / "libgda_san.so")
    _run(["g++", "-shared", "-fsanitize=address,undefined", "-o", lib_so, api_o,
          *[os.path.join(BUILD, o) for o in KERNEL_OBJS], "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    return d, oracle_so, lib_so


def test_harness_catches_a_planted_overflow(san_builds):
    d, _, _ = san_builds
    src = d / "overflow.c"
    src.write_text("#include <stdlib.h>\nint poke(int n, int i) { int* p = malloc(n * sizeof(int));"
                   " p[i] = 1; int r = p[0]; free(p); return r; }\n")
    so = str(d / "liboverflow.so")
    _run(["gcc", *SAN, "-fPIC", "-shared", "-o", so, str(src)])
    code = f"import ctypes; ctypes.CDLL({so!r}).poke(4, 4)"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       env=_env({}))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_oracle_pins_and_abi_under_sanitizers(san_builds):
    _, oracle_so, lib_so = san_builds
    probe = ("import oracle; from attention_gda_fwd_amd import _lib; "
             "print(oracle.LIB_PATH); print(_lib.LIB_PATH)")
    env = _env({"GDA_ORACLE_LIB": oracle_so, "GDA_LIB": lib_so})
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True, env=env,
                       cwd=ROOT)
    assert r.returncode == 0 and r.stdout.split() == [oracle_so, lib_so], r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", "tests/test_oracle_pins.py",
                        "tests/test_abi_cpu.py"], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
