"""AddressSanitizer + UndefinedBehaviorSanitizer builds, CPU only:
  * the whole CPU oracle (gcc, OpenMP) driven through every entry point on
    small ragged problems, leak checking on (tests/sanitize/oracle_driver.c);
  * the C ABI's host code -- argument checks, size and workspace queries,
    error text -- with the sanitizers on the host pass only (the launchers
    replaced by stand-ins; every call the driver makes must fail validation
    before any device work; tests/sanitize/abi_driver.cpp).
Each driver runs as a child process and must exit 0 with no sanitizer
report."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_attention_video_smooth_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="vc_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_oracle_under_asan_ubsan(tmp):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.fail("gcc not found")
    exe = os.path.join(tmp, "oracle_driver")
    _run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "vc_oracle.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = _run([exe], env=env, timeout=600)
    assert "oracle driver ok" in r.stdout and "runtime error" not in r.stderr


def test_abi_host_code_under_asan_ubsan(tmp):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc):
        pytest.fail("hipcc not found")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    base = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *inc, *HOST_SAN]
    objs = []
    for src, host_only, xhip in ((os.path.join(CSRC, "vc_abi.hip"), False, False),
                                 (os.path.join(CSRC, "vc_host.hip"), True, False),
                                 (os.path.join(HERE, "launch_stubs.cpp"), True, True),
                                 (os.path.join(HERE, "abi_driver.cpp"), True, True)):
        obj = os.path.join(tmp, os.path.basename(src) + ".o")
        _run(base + (["--offload-host-only"] if host_only else []) + (["-x", "hip"] if xhip else [])
             + ["-c", src, "-o", obj])
        objs.append(obj)
    exe = os.path.join(tmp, "abi_driver")
    _run([hipcc, "--offload-arch=gfx950", *HOST_SAN, *objs, "-o", exe])
    # the HIP runtime's own allocations are not this library's to check
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = _run([exe], env=env, timeout=300)
    assert "abi driver ok" in r.stdout and "runtime error" not in r.stderr
