"""Host AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only).

tests/native/build_sanitized.sh builds two programs: the library's argument
validation (ssd_api.hip, host code instrumented) driven through the C ABI by
abi_sanitize.c with calls that validation rejects, and the fp64 oracle's C
code driven by oracle_sanitize.c over small problems, ragged lengths, L = 0
and the backward pass.  Any out-of-bounds access, signed overflow, invalid
enum load or misaligned access aborts the program (no recovery)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OBJ = os.path.join(ROOT, "mamba_ssd_selective_amd", "_build")


@pytest.fixture(scope="module")
def programs(tmp_path_factory):
    if not os.path.exists(os.path.join(OBJ, "ssd_kernels.o")):
        pytest.fail("the library is not built; run __graft_entry__.build()")
    for tool in ("/opt/rocm/bin/hipcc", "/opt/rocm/llvm/bin/clang++"):
        if not os.path.exists(tool):
            pytest.skip("%s not found" % tool)
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    out = str(tmp_path_factory.mktemp("san"))
    r = subprocess.run([os.path.join(HERE, "native", "build_sanitized.sh"), out],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def _run(path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    return subprocess.run([path], capture_output=True, text=True, timeout=300, env=env)


def test_abi_validation_under_sanitizers(programs):
    r = _run(os.path.join(programs, "abi_san"))
    assert r.returncode == 0 and "abi sanitize: ok" in r.stdout, r.stdout + r.stderr


def test_oracle_under_sanitizers(programs):
    r = _run(os.path.join(programs, "oracle_san"))
    assert r.returncode == 0 and "oracle sanitize: ok" in r.stdout, r.stdout + r.stderr
