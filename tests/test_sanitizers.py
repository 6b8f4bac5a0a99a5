"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs, on the CPU.

1. The C oracle is rebuilt with gcc -fsanitize=address,undefined and every
   oracle pin test runs against that build (the pins call each oracle
   function, including packed sequences with empty ones, the reverse mode,
   the decode slot indirection and the preparation/epilogue paths).
2. The C-ABI layer (kda_api.cpp: argument validation, workspace sizing,
   status strings, the no-device path) is rebuilt with the host-side
   sanitizers and linked with the kernels of the normal build; the ABI and
   binding-check tests then run against it.

Each run is a child process with the sanitizer runtime preloaded (the Python
interpreter itself is not instrumented), leak checking off (the interpreter
keeps its allocations to the end), and any report fatal.  No GPU is used: the
ABI tests stop at host validation or at the device query.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_attention_sequence_chunkwise_amd")
HIPCC = "/opt/rocm/bin/hipcc"


def _run(tmp, preload, plugin_src, tests):
    with open(os.path.join(tmp, "sanitized_plugin.py"), "w") as f:
        f.write(plugin_src)
    env = dict(os.environ)
    env.update(LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=tmp + os.pathsep + ROOT)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "sanitized_plugin", "-p",
                        "no:cacheprovider", *tests], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime not available")
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fopenmp",
                           "-fPIC", "-shared", "-std=c99", "-o", lib,
                           os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm"])
    plugin = "import oracle\noracle._LIB = %r\nassert oracle._load()._name == %r\n" % (lib, lib)
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*pins.py")))
    assert len(tests) >= 5
    _run(str(tmp_path), asan, plugin, tests)


def test_abi_under_asan_ubsan(tmp_path):
    objs = [os.path.join(PKG, "_build", n + ".o") for n in ("kda_decode", "kda_prefill", "kda_dplr")]
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(HIPCC) or not rt or not all(os.path.exists(o) for o in objs):
        pytest.skip("hipcc, its AddressSanitizer runtime or the kernel objects are missing")
    obj = str(tmp_path / "kda_api_sanitized.o")
    lib = str(tmp_path / "libkda_sanitized.so")
    # host-side instrumentation only: every -fsanitize sits behind -Xarch_host
    cmd = [HIPCC, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-c", os.path.join(PKG, "csrc", "kda_api.cpp"), "-o", obj]
    subprocess.check_call(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, obj,
                           *objs], stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    plugin = ("import linear_attention_sequence_chunkwise_amd as kda\n"
              "assert kda.load_library(%r)._name == %r\n" % (lib, lib))
    _run(str(tmp_path), rt[0], plugin,
         [os.path.join(ROOT, "tests", "test_abi.py"),
          os.path.join(ROOT, "tests", "test_binding_checks.py")])
