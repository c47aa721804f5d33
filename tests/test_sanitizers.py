"""The CPU tier under AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (oracle/oracle.c) built with gcc -fsanitize=address,undefined runs
  every pin, and each planted mutant of it that changes indexing or layout,
  built the same way, must still be caught: a failing pin or a sanitizer
  report both count.
* The library's host code (the C ABI's validation in csrc/attn_api.hip and the
  launchers) built with host-only sanitizers (hipcc, -Xarch_host before each
  -fsanitize=; device code as usual) runs tests/test_abi.py and the
  property-based fuzz of the same validation, tests/test_abi_fuzz.py.

Python itself is not instrumented, so each run is a child process with the
sanitizer runtime of its compiler preloaded (gcc's libasan for the oracle,
clang's for hipcc's host code; entries already in LD_PRELOAD are kept).
Nothing here touches a GPU: every ABI call is refused before any HIP call.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle
from transformer_attention_flash_amd import build as hip_build
from test_oracle_mutants import MUTANTS, SRC as ORACLE_SRC

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
GCC_SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _gcc_asan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        path = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(path):
            return path
    return None


def _env(runtime):
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    return env


_PINS = """
import json, sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
from oracle_pins import ALL_PINS
orc = oracle.Oracle(oracle.load({lib!r}))
failed = []
for name, pin in ALL_PINS:
    try:
        pin(orc)
    except (AssertionError, ValueError, FloatingPointError):
        failed.append(name)
print(json.dumps(failed))
"""


def _run_pins(lib, runtime):
    code = _PINS.format(root=ROOT, tests=TESTS, lib=lib)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                          env=_env(runtime))


def _sanitizer_report(res):
    return "Sanitizer" in res.stderr or "runtime error:" in res.stderr


@pytest.fixture(scope="module")
def gcc_asan():
    path = _gcc_asan()
    if path is None:
        pytest.skip("gcc's libasan is not available")
    return path


def test_oracle_pins_clean_under_sanitizers(gcc_asan, tmp_path):
    lib = oracle.build(ORACLE_SRC, str(tmp_path / "liboracle_san.so"), GCC_SAN)
    res = _run_pins(lib, gcc_asan)
    assert res.returncode == 0 and not _sanitizer_report(res), res.stderr[-3000:]
    assert res.stdout.strip().splitlines()[-1] == "[]", f"pins failing under sanitizers: {res.stdout[-500:]}"


# The mutants whose mistake is in indexing or layout (where a sanitizer may see an access the
# pins do not); the arithmetic ones run unsanitized in test_oracle_mutants.py.
INDEXING = ("scatter_", "slot_copy_", "decode_", "cached_", "token_", "head_", "gqa_", "k_used", "v_index",
            "rows_entry")
SANITIZED_MUTANTS = [m for m in MUTANTS if m[0].startswith(INDEXING)]


@pytest.mark.parametrize("mid,old,new", SANITIZED_MUTANTS, ids=[m[0] for m in SANITIZED_MUTANTS])
def test_sanitized_mutant_is_caught(mid, old, new, gcc_asan, tmp_path):
    src = open(ORACLE_SRC).read()
    mutated = tmp_path / f"oracle_{mid}.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / f"liboracle_{mid}.so"), GCC_SAN)
    res = _run_pins(lib, gcc_asan)
    caught = res.returncode != 0 or _sanitizer_report(res) or res.stdout.strip().splitlines()[-1] != "[]"
    assert caught, f"sanitized mutant {mid} passed every pin"


def test_abi_clean_under_host_sanitizers(tmp_path):
    runtime = _clang_asan()
    if runtime is None or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or clang's ASan runtime is not available")
    lib = str(tmp_path / "libattn_san.so")
    hip_build.build(out=lib, extra_flags=HOST_SAN)
    code = ("import sys; sys.path[:0] = [{root!r}, {tests!r}]\n"
            "import transformer_attention_flash_amd as taf\n"
            "taf._LIB_PATH = {lib!r}\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {abi!r}, {fuzz!r}]))\n").format(
                root=ROOT, tests=TESTS, lib=lib, abi=os.path.join(TESTS, "test_abi.py"),
                fuzz=os.path.join(TESTS, "test_abi_fuzz.py"))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600,
                         env=_env(runtime))
    assert res.returncode == 0 and not _sanitizer_report(res), (res.stdout[-3000:], res.stderr[-3000:])
