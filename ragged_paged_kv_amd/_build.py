"""Build libcbattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python ragged_paged_kv_amd/_build.py [--debug-host]

Objects go to ``_build/`` at the repository root; the library is written next to this file.
``--debug-host`` adds host-side AddressSanitizer/UBSan (device code is never sanitised).
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
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libcbattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcbattn.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False, debug_host: bool = False) -> str:
    hipcc = _hipcc()
    obj_dir = os.path.join(ROOT, "_build", "debug" if debug_host else "release")
    os.makedirs(obj_dir, exist_ok=True)
    common = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              "-I", INCLUDE, "-I", CSRC,
              # packed fp32 VALU ops stay off: plain scalar fp32 code only
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    if debug_host:
        common += ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]

    def compile_one(src):
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        cmd = [hipcc] + common + ["-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd = [hipcc, "-x", "hip"] + common + ["-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources()))
    out = LIB_PATH if not debug_host else os.path.join(obj_dir, LIB_NAME)
    fd, tmp = tempfile.mkstemp(prefix=".libcbattn.", suffix=".so.tmp", dir=os.path.dirname(out))
    os.close(fd)
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if debug_host:
        link += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, debug_host="--debug-host" in sys.argv)
