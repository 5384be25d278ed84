"""CPU: the oracle and the C ABI's host-side code under AddressSanitizer and
UndefinedBehaviorSanitizer.

Each test builds an instrumented copy of a library into a temporary folder and
runs an existing CPU test file against it in a child process that preloads
the sanitizer runtime (the Python interpreter itself is not instrumented):

  * the oracle (plain C, gcc): every oracle pin;
  * libhisa with its host code instrumented (hipcc; the GPU code is built as
    usual and never runs here): the ABI tests -- every exported symbol, the
    workspace sizes and every argument check, which run on the host before
    anything would be enqueued.

Any invalid memory access or undefined behaviour aborts the child, so the
test fails.  Leak detection is off: the interpreter keeps its allocations.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def _run_child(code: str, preload: str, timeout: int):
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload, PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    return r.returncode, (r.stdout + r.stderr)[-6000:]


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = str(tmp_path / "libhisa_oracle_san.so")
    srcs = [os.path.join(ROOT, "oracle", f) for f in ("hisa_oracle.c", "attention_oracle.c")]
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-shared", "-fPIC", "-o", lib, *srcs, "-lm"], check=True)
    code = ("import sys, pytest; import oracle.oracle as o; o._LIB_PATH = %r; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_oracle_pins.py']))" % lib)
    rc, out = _run_child(code, f"{asan} {ubsan}", timeout=900)
    assert rc == 0, out
    assert " passed" in out


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/*/libclang_rt.asan*x86_64*.so"))
    hits = [h for h in hits if os.path.basename(h) in ("libclang_rt.asan-x86_64.so", "libclang_rt.asan.so")]
    return hits[-1] if hits else None


def test_abi_host_code_under_sanitizers(tmp_path):
    rt = _clang_asan_runtime()
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not rt or not os.path.exists(hipcc):
        pytest.skip("hipcc or clang's address-sanitizer runtime is not installed")
    from sparse_attention_token_amd import build as B

    objs = {s: os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES}
    if not all(os.path.exists(o) for o in objs.values()):
        B.build()
    # the ABI source with its host code instrumented; the other objects as built
    san = str(tmp_path / "hisa_abi_san.o")
    host_san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    r = subprocess.run([hipcc, *B.FLAGS, *host_san, "-c", os.path.join(B.CSRC, "hisa_abi.hip"), "-o", san],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    lib = str(tmp_path / "libhisa_san.so")
    others = [o for s, o in objs.items() if s != "hisa_abi.hip"]
    r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *host_san, "-o", lib, san, *others],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    code = ("import sys, pytest; from sparse_attention_token_amd import hisa; hisa._LIB_PATH = %r; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi_host.py']))" % lib)
    rc, out = _run_child(code, rt, timeout=600)
    assert rc == 0, out
    assert " passed" in out
