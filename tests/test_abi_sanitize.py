"""The host-side ABI checks under AddressSanitizer and UndefinedBehaviorSanitizer.

The validation code of the C ABI (argument checks, size arithmetic, overlap
tests, error strings) is rebuilt with the host half of hipcc instrumented
(`-Xarch_host -fsanitize=...`; device code is untouched) and linked with the
library's other objects.  Python itself is not instrumented, so the test
builds a small launcher that embeds the interpreter and carries the sanitizer
runtimes; it runs tests/test_abi_cpu.py with GDNQ_LIBRARY pointing at the
instrumented library.  Any sanitizer report fails the run.
"""

import os
import subprocess
import sysconfig

import pytest

from quantized_recurrent_state_gdnq_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _fresh_objects():
    """The library's objects under _build/, rebuilt when any is missing or
    older than a source or header it may include."""
    srcs = build.sources()
    hdrs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC) if f.endswith(".h")]
    hdrs.append(os.path.join(build.INCLUDE, "gdnq.h"))
    newest = max(os.path.getmtime(p) for p in srcs + hdrs)
    objs = [os.path.join(build.BUILD, os.path.basename(s) + ".o") for s in srcs]
    if not all(os.path.exists(o) and os.path.getmtime(o) >= newest for o in objs):
        build.build()
    return [o for o in objs if not o.endswith("abi.cpp.o")]


def test_abi_checks_under_asan_ubsan(tmp_path):
    inc = sysconfig.get_paths()["include"]
    libdir = sysconfig.get_config_var("LIBDIR")
    ldlib = sysconfig.get_config_var("LDLIBRARY") or ""
    if not (os.path.exists(CLANG) and os.path.exists(build.HIPCC)):
        pytest.skip("hipcc/clang not available")
    if not os.path.exists(os.path.join(inc, "Python.h")) or not ldlib.endswith(".so"):
        pytest.skip("no shared libpython to embed")
    objs = _fresh_objects()

    launcher = tmp_path / "pysan"
    src = tmp_path / "pysan.c"
    src.write_text("#include <Python.h>\nint main(int argc, char** argv) { return Py_BytesMain(argc, argv); }\n")
    pylib = ldlib[3:-3]  # libpython3.10.so -> python3.10
    _run([CLANG, "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-I", inc, str(src),
          "-L", libdir, f"-l{pylib}", "-o", str(launcher)])

    obj = tmp_path / "abi_san.o"
    _run([build.HIPCC, "-O1", "-g"] + [f for f in build.COMMON if f != "-O3"] + build.GPU_FLAGS + SAN +
         ["-c", os.path.join(build.CSRC, "abi.cpp"), "-o", str(obj)])
    syms = _run(["nm", "-u", str(obj)]).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms  # the host code is instrumented
    lib = tmp_path / "libgdnq_san.so"
    _run([build.HIPCC, f"--offload-arch={build.ARCH}", "-shared", "-fPIC"] + SAN[:4] +
         ["-o", str(lib), str(obj)] + objs)

    env = dict(os.environ)
    env.update(GDNQ_LIBRARY=str(lib), PYTHONPATH=ROOT,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the instrumented library is the one the binding loads
    r = _run([str(launcher), "-c",
              "from quantized_recurrent_state_gdnq_amd import _lib; "
              "print(_lib.LIB_PATH); print(open('/proc/self/maps').read().count('libgdnq_san.so') > 0)"],
             env=env, cwd=ROOT, timeout=300)
    assert r.stdout.split() == [str(lib), "True"], r.stdout
    r = subprocess.run([str(launcher), "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert " passed" in out and "failed" not in out, out[-3000:]
