"""Builds libpkv.so (HIP for gfx950) in the package directory.

    python paged_kv_cache_amd/build.py [-i] [-v]
    python paged_kv_cache_amd/build.py --sanitize     (host runtime under ASan/UBSan)

(run as a script: importing the package loads the library this builds)

compiles csrc/*.hip and csrc/*.cpp with hipcc into objects under
``_build/`` and links them into ``paged_kv_cache_amd/libpkv.so``. All device
code is built with ``-target-feature -packed-fp32-ops`` (no packed fp32
arithmetic is generated) and with the matrix-core instructions in their
VGPR form (``-amdgpu-mfma-vgpr-form``): the attention kernels' accumulators
then live in ordinary VGPRs instead of being copied between AGPRs and VGPRs
around every online-softmax rescale, which frees registers for occupancy.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv)")


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def compile_cmd(src: str, obj: str):
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Wall", "-Wno-unused-function", "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    return cmd


def _stale(src: str, obj: str) -> bool:
    if not os.path.exists(obj):
        return True
    deps = [src] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".h", ".hpp"))]
    deps.append(os.path.join(ROOT, "include", "pkv.h"))
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compiles every source (with ``incremental``, only those whose object
    is older than the source or any header) and links libpkv.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = []
    for s in srcs:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append((os.path.join(CSRC, s), obj))
    todo = [j for j in jobs if not incremental or _stale(*j)]

    def run(job):
        src, obj = job
        cmd = compile_cmd(src, obj)
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        return src, r.returncode, out

    with ThreadPoolExecutor(max_workers=max(1, min(8, len(todo)))) as ex:
        results = list(ex.map(run, todo))
    bad = [(s, out) for s, rc, out in results if rc != 0]
    for s, rc, out in results:
        if out.strip() and (verbose or rc != 0):
            print(f"--- {os.path.basename(s)}\n{out}", file=sys.stderr)
    if bad:
        raise RuntimeError("libpkv build failed: " + ", ".join(os.path.basename(s) for s, _ in bad))
    tmp = LIB + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for _, o in jobs]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libpkv link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libpkv_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def build_sanitized(verbose: bool = False) -> str:
    """A debug build of the host runtime for CPU-only checking: the C++
    sources (pool, planner, C ABI) compiled by g++ with AddressSanitizer and
    UndefinedBehaviorSanitizer and with PKV_CHECKS (the planner aborts if a
    write would land in a block that has another holder), linked with the
    ordinary device object of kernels.hip (no sanitizer in device code) into
    ``_build/san/libpkv_san.so``. Load it with PKV_LIBRARY pointing at it and
    the sanitizer runtime preloaded (see README)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    # objects in a directory of this process's own, the library renamed into
    # place: concurrent builds (parallel test workers) do not mix their files
    work = tempfile.mkdtemp(dir=SAN_DIR)
    objs = []
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for s in sources():
        src = os.path.join(CSRC, s)
        if s.endswith(".hip"):
            # the device code as in the ordinary build (reused if up to date)
            obj = os.path.join(BUILD, s + ".o")
            if _stale(src, obj):
                r = subprocess.run(compile_cmd(src, obj), capture_output=True, text=True)
                if r.returncode != 0:
                    raise RuntimeError(f"{s}: " + r.stdout + r.stderr)
            objs.append(obj)
            continue
        obj = os.path.join(work, s + ".o")
        cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fPIC",
               "-D__HIP_PLATFORM_AMD__", "-DPKV_CHECKS", "-I" + os.path.join(rocm, "include"),
               "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *SAN_FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0 or (verbose and (r.stdout or r.stderr)):
            print(f"--- {s}\n{r.stdout}{r.stderr}", file=sys.stderr)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build of {s} failed")
        objs.append(obj)
    tmp = os.path.join(work, "libpkv_san.so")
    link = ["g++", "-shared", *SAN_FLAGS, "-o", tmp, *objs,
            "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitizer link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, SAN_LIB)
    shutil.rmtree(work, ignore_errors=True)
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of g++'s AddressSanitizer runtime (to preload into Python)."""
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv, incremental="-i" in sys.argv))
