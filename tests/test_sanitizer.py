"""The host runtime (block pool, persistent tables, append planner, attention
planner, C ABI argument checks) under AddressSanitizer and
UndefinedBehaviorSanitizer, with the debug check that aborts if the planner
would write into a block another holder still reads (a block being written
is never aliased: Dendrite author's reply, "Why Rust?").

The sanitizer build (``build.py --sanitize``) compiles the C++ sources with
g++ and links the ordinary device object; the table tests and the plain-C
ABI program then run against it on the CPU. No GPU is touched."""

from __future__ import annotations

import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="g++/gcc not installed")


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "pkv_build", os.path.join(ROOT, "paged_kv_cache_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def san():
    b = _build_module()
    lib = b.build_sanitized()
    env = dict(os.environ)
    env.update(PKV_LIBRARY=lib, LD_PRELOAD=b.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return lib, env


def test_table_tests_clean_under_sanitizers(san):
    _, env = san
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_pool.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail


def test_c_program_clean_under_sanitizers(san, tmp_path):
    lib, env = san
    exe = str(tmp_path / "abi_host_san")
    cmd = ["gcc", "-std=c11", "-g", "-fsanitize=address,undefined", "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), lib, "-Wl,-rpath," + os.path.dirname(lib),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = {k: v for k, v in env.items() if k != "LD_PRELOAD"}  # linked in, not preloaded
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
