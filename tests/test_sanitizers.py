"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C oracle built with gcc ``-fsanitize=address,undefined`` (reports abort)
  runs every oracle pin and the workload tests, in a child process with gcc's
  libasan and libubsan preloaded.
* The HIP library built with its host code instrumented
  (``-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined``; device
  code is not instrumented) runs the ABI and binding tests (argument checks,
  error paths, exported symbols), in a child process with clang's ASan
  runtime preloaded.

Both builds go to a temporary directory. The same runs by hand::

    python -c "import oracle; oracle.build(sanitize=True, out='/tmp/o.so')"
    LD_PRELOAD=$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so) \\
        ASAN_OPTIONS=detect_leaks=0 python ... (see _run below)
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(preload, setup, files, tmp_path):
    script = (
        "import sys\n"
        f"sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, 'tests')!r}]\n"
        f"{setup}\n"
        "import pytest\n"
        f"sys.exit(pytest.main({files!r} + ['-q', '-x', '-p', 'no:cacheprovider']))\n")
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", script], cwd=tmp_path, env=env,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout


def _symbols(lib):
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    return out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    import oracle
    lib = oracle.build(sanitize=True, out=str(tmp_path / "liboracle_sanitized.so"))
    assert "__asan" in _symbols(lib) and "__ubsan" in _symbols(lib)
    preload = ":".join(subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
                       for n in ("libasan.so", "libubsan.so"))
    files = sorted(f for f in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))
                   if "mutants" not in f) + [os.path.join(ROOT, "tests", "test_workloads.py")]
    _run(preload, f"import oracle\noracle.use_library({lib!r})", files, tmp_path)


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    from sparse_attention_kv_hisparse_amd.build import build
    lib = build(sanitize=True, out=str(tmp_path / "libhisparse_sanitized.so"))
    assert "__asan" in _symbols(lib) and "__ubsan" in _symbols(lib)
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts:
        pytest.skip("clang's ASan runtime is not installed")
    files = [os.path.join(ROOT, "tests", "test_abi.py"),
             os.path.join(ROOT, "tests", "test_binding_shapes.py")]
    _run(rts[0], f"from sparse_attention_kv_hisparse_amd import _lib\n_lib.load({lib!r})",
         files, tmp_path)
