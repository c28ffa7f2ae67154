"""CPU sanitizer build of the oracle and the input generator.

tests/native/sanitize_driver.c calls every exported function of
oracle/oracle.c and fixtures/gen.c on small edge-case inputs. It is built
here with gcc, AddressSanitizer and UndefinedBehaviorSanitizer (runtimes
linked into the executable, every report fatal) and must finish cleanly: no
out-of-bounds access, use after free, leak, signed overflow, misaligned or
out-of-range conversion anywhere in the checker code the parity tests rely on.
No GPU code is built or run here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "tests", "native", "sanitize_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "fixtures", "gen.c")]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-static-libasan", "-static-libubsan"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.fail("gcc is required for the sanitizer build")
    exe = str(tmp_path_factory.mktemp("san") / "sanitize_driver")
    cmd = ["gcc", "-std=c11", "-O1", "-g", *SAN, "-fopenmp", *SOURCES, "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_oracle_and_generator_clean_under_asan_ubsan(driver):
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
