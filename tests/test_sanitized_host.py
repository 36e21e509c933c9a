"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

A copy of the repository's Python sources, tests and C / HIP sources is built
into a scratch tree with the sanitizers on the host side, and the CPU tests run
there in a child process with the sanitizer runtime preloaded:

* the oracle (oracle/oracle.c, gcc -fsanitize=address,undefined): every oracle
  pin (tests/test_oracle_*.py) and the bench's oracle leg (test_bench_host.py);
* libfq.so's host code (hipcc, the sanitizers on the host pass only; device code
  is built as usual and never runs here): the argument checks of every entry
  point (test_abi.py) and the binding's guards (test_bench_host.py).

Any sanitizer report aborts the child, so a non-zero exit fails the test.  No
kernel is launched: there is no GPU here, and every call that reaches the
library is rejected by its argument checks or goes to a recorder.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# the sanitizers on the host pass only: each -fsanitize right after -Xarch_host
HOST_SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=all -Xarch_host -shared-libasan").split()
ORACLE_SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV_SAN = dict(ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _copy_tree(dst):
    for sub in ("fake_quant_amd", "oracle", "tests", "include"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(dst, sub),
                        ignore=shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__", "*.pyc"))
    shutil.copy(os.path.join(ROOT, "bench.py"), dst)


def _run(cmd, cwd, env=None, timeout=900):
    res = subprocess.run(cmd, cwd=cwd, env=env, capture_output=True, text=True, timeout=timeout)
    assert res.returncode == 0, f"{cmd[:3]} failed ({res.returncode}):\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}"
    return res


def _sanitizer_is_live(tree, preload, probe):
    """A caller mistake planted on the CPU (a write past a small host array) must
    be reported, so the preloaded runtime and the instrumented build are active."""
    env = dict(os.environ, LD_PRELOAD=preload, **ENV_SAN)
    res = subprocess.run([sys.executable, "-c", probe], cwd=tree, env=env, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0 and "AddressSanitizer" in res.stderr, (res.returncode, res.stderr[-2000:])


def _pytest(tree, files, preload):
    env = dict(os.environ, LD_PRELOAD=preload, **ENV_SAN)
    res = _run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *files],
               cwd=tree, env=env)
    assert " passed" in res.stdout and "failed" not in res.stdout, res.stdout[-2000:]
    return res


def _oracle_build(tree, extra):
    from oracle import oracle as orc
    src = os.path.join(tree, "oracle", "oracle.c")
    _run(["gcc", *orc.CFLAGS, *extra, "-o", os.path.join(tree, "oracle", "liboracle.so"), src, "-lm"], cwd=tree)


@pytest.fixture(scope="module")
def tree(tmp_path_factory):
    if shutil.which("gcc") is None or not os.path.exists(HIPCC):
        pytest.skip("needs gcc and hipcc")
    t = str(tmp_path_factory.mktemp("sanitized"))
    _copy_tree(t)
    # the product library as built, for the oracle run (the host-code run below
    # replaces it with the sanitized build)
    lib = os.path.join(ROOT, "fake_quant_amd", "libfq.so")
    if not os.path.exists(lib):
        from fake_quant_amd import build as fqbuild
        fqbuild.build()
    shutil.copy(lib, os.path.join(t, "fake_quant_amd", "libfq.so"))
    return t


def test_oracle_under_sanitizers(tree):
    _oracle_build(tree, ORACLE_SANITIZE)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    _sanitizer_is_live(tree, libasan, "import numpy as np; from oracle import oracle as o; x = np.zeros(10, np.float32); "
                                      "o.lib().orc_ste_backward(o._ptr(x), o._ptr(x), 12, -1.0, 1.0, o._ptr(x))")
    files = sorted(os.path.relpath(p, tree) for p in glob.glob(os.path.join(tree, "tests", "test_oracle_*.py")))
    _pytest(tree, files + ["tests/test_bench_host.py"], libasan)


def test_library_host_code_under_sanitizers(tree):
    # the oracle without sanitizers here: one sanitizer runtime per process
    _oracle_build(tree, [])
    from fake_quant_amd import build as fqbuild
    csrc = os.path.join(tree, "fake_quant_amd", "csrc")
    flags = [f for f in fqbuild.FLAGS if f != "-O3"] + ["-O1", "-g", *HOST_SANITIZE]
    out = os.path.join(tree, "fake_quant_amd", "libfq.so")
    _run([HIPCC, *flags, "-I", os.path.join(tree, "include"), "-I", csrc, "-o", out,
          *sorted(glob.glob(os.path.join(csrc, "*.hip")))], cwd=tree)
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("clang's shared ASan runtime is not installed")
    _sanitizer_is_live(tree, rt[0], "import numpy as np; from fake_quant_amd import fq; b = np.zeros(1, np.uint8); "
                                    "p = b.ctypes.data; fq.lib().fq_q4dq_sizes(100, p, p, p)")
    _pytest(tree, ["tests/test_abi.py", "tests/test_bench_host.py"], rt[0])
