"""The oracle's C part under AddressSanitizer and UndefinedBehaviorSanitizer.

A copy of oracle/ (with the pin tests and their fixtures) is built with
gcc -fsanitize=address,undefined, every report fatal, and the pins and the
property tests run against it in a separate process with the sanitizer
runtime preloaded.  Any out-of-bounds access, use of uninitialised stack
memory through an index, signed overflow or invalid shift in oracle.c fails
the test.  CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
             "-g", "-O1"]

CONFTEST = '''import os, sys
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import pytest
def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a GPU")
    config.addinivalue_line("markers", "slow: slow")
@pytest.fixture(scope="session")
def olib():
    import oracle
    return oracle.lib()
'''


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc AddressSanitizer runtime not installed")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    d = str(tmp_path / "san")
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    os.makedirs(os.path.join(d, "tests"))
    open(os.path.join(d, "tests", "conftest.py"), "w").write(CONFTEST)
    open(os.path.join(d, "tests", "__init__.py"), "w").close()
    for f in ("test_oracle_pins.py", "test_oracle_properties.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(d, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    os.makedirs(os.path.join(d, "token_routing_shuffle_amd"))
    for f in ("__init__.py", "workload.py"):
        shutil.copy(os.path.join(ROOT, "token_routing_shuffle_amd", f),
                    os.path.join(d, "token_routing_shuffle_amd", f))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), os.path.join(d, "pytest.ini"))
    b = subprocess.run([sys.executable, os.path.join(d, "oracle", "build.py"), *SAN_FLAGS],
                       capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1",
               LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_properties.py"],
                       cwd=d, capture_output=True, text=True, env=env, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]
    assert " passed" in r.stdout
