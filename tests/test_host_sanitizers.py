"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The oracle and the library's host side (ds_sel.cpp: argument checks, sizes,
capacity and no-device paths) are rebuilt with both sanitizers; the GPU
kernels' objects are linked as built, without them.  A child process that
preloads the sanitizer runtime then runs the oracle's pins and the C-ABI tests
against those builds; any sanitizer report fails the test.  Leak checking is
off: the Python interpreter itself is not leak-clean."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = "/opt/rocm/bin/hipcc"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(map(str, cmd))}\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    return res


@pytest.mark.slow
def test_host_code_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(CLANG) and os.path.exists(HIPCC)):
        pytest.skip("the ROCm clang toolchain is not installed")
    runtime = _run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    assert os.path.exists(runtime), runtime

    import oracle
    ora = tmp_path / "libds_sel_oracle_san.so"
    _run([CLANG, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
          "-o", str(ora), oracle.SOURCE, "-lm"])

    from sparse_attention_block_ds_amd import build
    kernels = [os.path.join(build.BUILD_DIR, s + ".o") for s in build.SOURCES if s != "ds_sel.cpp"]
    stale = any(not os.path.exists(o) or os.path.getmtime(o) < max(
        os.path.getmtime(os.path.join(build.CSRC, f)) for f in os.listdir(build.CSRC)) for o in kernels)
    if stale:
        build.build(verbose=False)  # the kernels' objects, current
    host_obj = tmp_path / "ds_sel_san.o"
    _run([HIPCC, *build.CXXFLAGS, "-O1", "-g", *HOST_SAN, "-x", "hip", "-c",
          os.path.join(build.CSRC, "ds_sel.cpp"), "-o", str(host_obj)])
    lib = tmp_path / "libdssel_san.so"
    _run([HIPCC, f"--offload-arch={build.ARCH}", "-shared", "-fPIC", "-o", str(lib), str(host_obj),
          *kernels])

    for built in (ora, lib):  # both really carry the instrumentation
        syms = _run(["nm", "-D", "--undefined-only", str(built)]).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, built

    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               DS_SEL_TEST_LIBRARY=str(lib), DS_SEL_TEST_ORACLE=str(ora))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "tests/test_abi_cpu.py", "tests/test_oracle.py", "-m", "not gpu",
                          "-k", "not struct_layout and not exports"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert res.returncode == 0, out[-6000:]
    assert " passed" in res.stdout
