"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two instrumented builds, each run under the CPU tests that drive it, in a
child process with the matching sanitizer runtime preloaded (the Python
interpreter itself is not instrumented):

* the oracle (oracle/q8kv_oracle.c), built by gcc with
  -fsanitize=address,undefined, under every oracle test (the pins, the
  mutation battery, the trace and split forms);
* the library (csrc/q8kv.hip) with its host code built by hipcc with the same
  two sanitizers (device code as usual), under the ABI tests: argument
  validation of every entry point and the partition plan.  No test there
  makes a HIP call.

Undefined behaviour halts the run (no recovery), as does any ASan report;
leak checking is off (the interpreter's own allocations would drown it).
A canary library with a one-past-the-end heap read, loaded the same way,
first shows that each setup reports errors at all.
"""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}
CANARY = textwrap.dedent("""
    #include <stdlib.h>
    int canary_read_past_end(int n) {
        int* p = (int*)malloc(sizeof(int) * n);
        for (int i = 0; i < n; ++i) p[i] = i;
        int r = p[n];
        free(p);
        return r;
    }
""")


def gcc_runtime():
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def clang_runtime():
    found = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                   "libclang_rt.asan-x86_64.so"))
    return found[0] if found else None


def child(code_or_args, preload, extra_env, timeout=600):
    env = dict(os.environ, **SAN_ENV, **extra_env, LD_PRELOAD=preload)
    env.pop("PYTEST_ADDOPTS", None)
    args = code_or_args if isinstance(code_or_args, list) else ["-c", code_or_args]
    return subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def canary_call(lib):
    return f"import ctypes; print(ctypes.CDLL({lib!r}).canary_read_past_end(4))"


@pytest.fixture(scope="module")
def work(tmp_path_factory):
    return tmp_path_factory.mktemp("san")


def test_oracle_under_asan_ubsan(work):
    rt = gcc_runtime()
    if not os.path.isabs(rt):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-fPIC", "-shared"]
    # the canary: the setup must report a heap overflow
    src = work / "canary.c"
    src.write_text(CANARY)
    subprocess.run(["gcc"] + flags + [str(src), "-o", str(work / "libcanary_gcc.so")], check=True)
    r = child(canary_call(str(work / "libcanary_gcc.so")), rt, {})
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
    # the oracle, with its own flags plus the sanitizers
    lib = work / "liboracle_san.so"
    subprocess.run(["gcc"] + flags + ["-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11",
                                      "-Wall", "-Wextra", os.path.join(ROOT, "oracle", "q8kv_oracle.c"),
                                      "-o", str(lib), "-lm"], check=True)
    env = {"Q8KV_ORACLE_LIB": str(lib)}
    r = child("import oracle; print(oracle._load()._name)", rt, env)
    assert r.returncode == 0 and r.stdout.strip() == str(lib), r.stderr[-2000:]
    r = child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
               "tests/test_oracle_quant.py", "tests/test_oracle_decode.py", "tests/test_oracle_append_decode.py",
               "tests/test_oracle_fp8.py", "tests/test_oracle_q40.py", "tests/test_oracle_quest.py",
               "tests/test_oracle_mutants.py"], rt, env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr


def test_library_host_code_under_asan_ubsan(work):
    rt = clang_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime under ROCM_PATH")
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    # the canary, through the same runtime
    src = work / "canary.c"
    src.write_text(CANARY)
    subprocess.run([clang, "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address", "-shared-libasan",
                    str(src), "-o", str(work / "libcanary_clang.so")], check=True)
    r = child(canary_call(str(work / "libcanary_clang.so")), rt, {})
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
    # the library: the usual flags, host code instrumented
    sys.path.insert(0, ROOT)
    try:
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_q8kv_build_for_san", os.path.join(ROOT, "decode_attention_int8_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
    finally:
        sys.path.pop(0)
    flags = [f for f in b.FLAGS if f != "-O3"] + ["-O1", "-g"] + host_san + ["-shared-libasan"]
    lib = work / "libq8kv_san.so"
    res = subprocess.run([hipcc] + flags + [b.SRC, "-o", str(lib)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = {"Q8KV_LIBRARY": str(lib)}
    r = child("import decode_attention_int8_amd as q8; print(q8.lib._name)", rt, env)
    assert r.returncode == 0 and r.stdout.strip().endswith(str(lib)), r.stderr[-2000:]
    r = child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", "tests/test_abi.py"], rt, env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
