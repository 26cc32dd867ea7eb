"""Build libkvfuse.so (gfx950) from the HIP sources in this directory.

    python -m rag_kv_cache_kvf_amd.csrc.build [--jobs N]

Every .hip file is compiled to an object under <repo>/_build/ with hipcc and
the objects are linked into rag_kv_cache_kvf_amd/libkvfuse.so.  The build
always recompiles (it is the "does it build" check); it never needs a GPU.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
OUT_LIB = os.path.join(PKG, "libkvfuse.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
    # packed fp32 instructions stay off (plain scalar fp32 code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", HERE,
    # per-kernel register / scratch report, checked below
    "-Rpass-analysis=kernel-resource-usage",
]

# A kernel whose private arrays the compiler could not keep in registers runs
# them through scratch memory, an order of magnitude slower; a few spilled
# dwords are tolerable, a demoted accumulator array is not.
MAX_SCRATCH_BYTES = 64
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]):\s+(\S+)")


def _resources(stderr: str) -> dict:
    """kernel name -> {VGPRs, AGPRs, ScratchSize, Occupancy} from the remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(stderr):
        key, val = m.group(1).split(" ")[0], m.group(2)
        if key == "Function":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val)
    return out


# per-file code-generation options
FILE_FLAGS = {
    # the attention kernel runs one wave per SIMD with its score accumulators
    # feeding VALU softmax: keep MFMA results in VGPRs instead of AGPRs (no
    # accumulator copies); spills go to the otherwise unused AGPRs
    "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def sources():
    return sorted(glob.glob(os.path.join(HERE, "*.hip")) + glob.glob(os.path.join(HERE, "kernels", "*.hip")))


def _compile(src: str, out_dir: str = BUILD_DIR, extra: tuple = ()) -> str:
    rel = os.path.relpath(src, HERE).replace(os.sep, "_")
    obj = os.path.join(out_dir, rel[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    res = _resources(r.stderr)
    bad = {k: v for k, v in res.items() if v.get("ScratchSize", 0) > MAX_SCRATCH_BYTES}
    if bad:
        raise RuntimeError(f"kernels in {src} use scratch memory beyond {MAX_SCRATCH_BYTES} B/lane: {bad}")
    with open(obj[:-2] + ".resources.txt", "w") as f:
        for k, v in sorted(res.items()):
            f.write(f"{k} {v}\n")
    # keep real diagnostics, drop the resource remarks and the host pass's
    # note about the GPU-only feature
    noise = "'-packed-fp32-ops' is not a recognized feature"
    lines = r.stderr.splitlines()
    keep, skip = [], False
    for l in lines:
        if "remark:" in l:
            skip = True          # the remark and its source-excerpt lines
            continue
        if skip and (l.startswith(" ") or l.strip() == ""):
            continue
        skip = False
        if noise not in l and "warning generated" not in l and "warnings generated" not in l:
            keep.append(l)
    warn = "\n".join(keep).strip()
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT_LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # A kernel template whose host-side instantiation fails (for instance a
    # device builtin called with an implicit narrowing conversion) loses its
    # launch stub without any diagnostic; the library would then not load.
    r = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError(f"kernel launch stubs missing from the library: {missing}")
    shutil.move(tmp, OUT_LIB)
    if verbose:
        print(f"built {OUT_LIB} from {len(srcs)} sources")
    return OUT_LIB


# AddressSanitizer on the host code only: each -fsanitize= right after
# -Xarch_host, so the device code is built exactly as in the library.
ASAN_HOST = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g")
ASAN_DIR = os.path.join(BUILD_DIR, "asan")
CLANG = os.environ.get("KVF_CLANG", "/opt/rocm/llvm/bin/clang")


def build_asan(driver_src: str, jobs: int | None = None) -> str:
    """A host-AddressSanitizer build of the library (_build/asan/libkvfuse_asan.so)
    and of a C test driver linked against it; returns the driver's path.
    For checking the host-side validation and bookkeeping on a machine
    without a GPU."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, ASAN_DIR, ASAN_HOST), srcs))
    lib = os.path.join(ASAN_DIR, "libkvfuse_asan.so")
    # the sanitizer runtime comes from the driver executable (statically
    # linked there), which resolves the library's instrumentation calls
    r = subprocess.run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-Xarch_host",
                        "-fsanitize=address", "-o", lib, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"asan link failed:\n{r.stdout}\n{r.stderr}")
    exe = os.path.join(ASAN_DIR, os.path.splitext(os.path.basename(driver_src))[0])
    r = subprocess.run([CLANG, "-fsanitize=address", "-fno-omit-frame-pointer",
                        "-g", "-O1", "-I", INCLUDE, driver_src, "-o", exe, "-L", ASAN_DIR,
                        "-lkvfuse_asan", f"-Wl,-rpath,{ASAN_DIR}"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"asan driver build failed:\n{r.stdout}\n{r.stderr}")
    return exe


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    build(ap.parse_args().jobs)
