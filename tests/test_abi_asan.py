"""The C ABI's host code under sanitizers (CPU only): the ABI tests run in a child
process against a copy of the library whose host code is instrumented with
AddressSanitizer or UndefinedBehaviorSanitizer (argument validation, the ring drivers'
host loops, positions and pair counts); any sanitizer report fails the child.  The child
runs without output capture (-s), so a sanitizer that ends it still gets its report into
the failure message."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    if shutil.which("g++") is None:
        return None
    path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(600)
def test_abi_suite_under_host_asan(tmp_path):
    rt = _libasan()
    if rt is None:
        pytest.skip("no g++ AddressSanitizer runtime on this host")
    sys.path.insert(0, ROOT)
    from ring_context_parallelism_amd.build import build_host_asan
    lib = build_host_asan(str(tmp_path / "libra_asan.so"))
    plugin = tmp_path / "asan_lib_plugin.py"
    plugin.write_text("import ring_context_parallelism_amd.ra as ra\n"
                      f"ra.LIB_PATH = {lib!r}\nra._lib = None\n")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT, os.environ.get("PYTHONPATH", "")]))
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-x", "-s", "-p", "asan_lib_plugin", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out


@pytest.mark.timeout(600)
def test_abi_suite_under_host_ubsan(tmp_path):
    """The same ABI tests against host code built with UndefinedBehaviorSanitizer, which
    aborts on the first report: signed overflow in the size and stride arithmetic of the
    validation, shifts, misaligned or null accesses in the drivers' host loops."""
    if shutil.which("g++") is None:
        pytest.skip("no g++ on this host")
    sys.path.insert(0, ROOT)
    from ring_context_parallelism_amd.build import build_host_sanitized
    try:
        lib = build_host_sanitized(str(tmp_path / "libra_ubsan.so"), "undefined")
    except subprocess.CalledProcessError:
        pytest.skip("g++ cannot build with UndefinedBehaviorSanitizer here")
    plugin = tmp_path / "ubsan_lib_plugin.py"
    plugin.write_text("import ring_context_parallelism_amd.ra as ra\n"
                      f"ra.LIB_PATH = {lib!r}\nra._lib = None\n")
    env = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT, os.environ.get("PYTHONPATH", "")]))
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-x", "-s", "-p", "ubsan_lib_plugin", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    out = r.stdout + r.stderr
    assert "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
