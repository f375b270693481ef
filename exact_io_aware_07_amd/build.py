"""Compile the HIP sources into exact_io_aware_07_amd/libattn.so for gfx950.

Run as `python -m exact_io_aware_07_amd.build` (or through __graft_entry__.build()).
Objects go to _build/ at the repository root; the shared library is written
next to this file so that it ships with the source tree.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_fp8.hip", "attn_ceiling.hip", "attn_api.hip"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for device code on purpose.
HIPFLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libattn.so")
    return path


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + HIPFLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    return obj, msgs


def build(verbose=False, extra_flags=(), out=LIB):
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, m in results:
            if m.strip():
                print(m)
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
