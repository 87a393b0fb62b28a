"""The C ABI from plain C: include/pkv.h compiles as C11 (-Wall -Wextra
-pedantic -Werror) and a host-only program linked against libpkv.so runs
the table verbs (fork, copy-on-write append planning, truncation, prompt
cache, free, error codes) as documented. No GPU: host calls only."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "paged_kv_cache_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_header_and_host_verbs_from_c(pkv, tmp_path):
    exe = str(tmp_path / "abi_host")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_host.c"),
           "-L" + LIB_DIR, "-lpkv", "-Wl,-rpath," + LIB_DIR, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
