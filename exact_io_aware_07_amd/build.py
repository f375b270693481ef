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
# Check build for the tests: the forward kernel with one LDS stage (tiles are
# loaded only after every wave has finished the previous one); its results must
# equal libattn.so's bit for bit.
LIB_SINGLE_STAGE = os.path.join(PKG, "libattn_single_stage.so")
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


def _compile(src, extra, obj_name=None):
    obj = os.path.join(BUILD, obj_name or os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + HIPFLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    return obj, msgs


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)


def build(verbose=False, extra_flags=(), out=LIB, single_stage=True):
    """Compile every source into `out`; with single_stage, also link the
    single-stage check library (the forward kernel rebuilt with one LDS stage)."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags)
    jobs = [(s, extra, None) for s in SOURCES]
    if single_stage:
        jobs.append(("attn_fwd.hip", extra + ["-DATTN_FWD_SINGLE_STAGE=1"], "attn_fwd_single_stage.o"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        results = list(ex.map(lambda j: _compile(*j), jobs))
    objs = [o for o, _ in results[:len(SOURCES)]]
    if verbose:
        for _, m in results:
            if m.strip():
                print(m)
    _link(objs, out)
    if verbose:
        print(f"built {out}")
    if single_stage:
        ss = [results[-1][0] if os.path.basename(o) == "attn_fwd.o" else o for o in objs]
        _link(ss, LIB_SINGLE_STAGE)
        if verbose:
            print(f"built {LIB_SINGLE_STAGE}")
    return out


def asan_runtime():
    """The clang AddressSanitizer runtime shipped with the HIP toolchain."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/lib/llvm")
    return hits[-1]


def build_asan(verbose=False):
    """Host code instrumented with AddressSanitizer (device code unchanged), into
    _build/asan/libattn_asan.so, for running the host-side ABI checks; load it
    with the runtime preloaded (LD_PRELOAD=asan_runtime())."""
    out_dir = os.path.join(BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    flags = "-O1 -g -Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()
    base = [f for f in HIPFLAGS if f != "-O3"]

    def comp(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([hipcc()] + base + flags + ["-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (asan) failed for {src}:\n{r.stderr[-4000:]}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(comp, SOURCES))
    out = os.path.join(out_dir, "libattn_asan.so")
    link = "-shared -fPIC -Xarch_host -fsanitize=address".split()
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}"] + link + objs + ["-o", out], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (asan) failed:\n{r.stderr[-4000:]}")
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
