"""Build libfd.so (the HIP library behind include/fd.h) for gfx950, in-tree.

    python -m decode_attention_03_amd.build

Each source compiles to an object under _build/ in parallel with hipcc, then
the objects link into decode_attention_03_amd/libfd.so.  Every call rebuilds.
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import json
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfd.so")
SOURCES = ["fd_api.cpp", "split_valu.hip", "split_mfma.hip", "combine.hip", "noalloc.hip"]
ARCH = "gfx950"

#: the source files each kernel family is compiled from; a measurement taken
#: on a kernel stays valid while these files are unchanged
KERNEL_SOURCES = {
    "split_valu": ["split_valu.hip", "partition.h", "partition_plan.h", "dev_common.h",
                   "fd_internal.h", "mfma_policy.h"],
    "split_mfma": ["split_mfma.hip", "partition.h", "partition_plan.h", "dev_common.h",
                   "fd_internal.h", "mfma_policy.h"],
    "combine": ["combine.hip", "partition.h", "partition_plan.h", "dev_common.h",
                "fd_internal.h", "mfma_policy.h"],
}


def source_hash(kernel: str) -> str:
    """Short SHA-256 over the sources of one kernel family."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


#: written beside the library: the hash of the sources it was built from
RECORD = os.path.join(PKG, "libfd.build.json")


def library_source_hash() -> str:
    """Short SHA-256 over every file the library is built from (csrc/ and
    include/), names included, so a build can be matched to its sources."""
    h = hashlib.sha256()
    for folder in (CSRC, os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(folder)):
            path = os.path.join(folder, name)
            if os.path.isfile(path):
                h.update(name.encode() + b"\0")
                with open(path, "rb") as f:
                    h.update(f.read())
    return h.hexdigest()[:16]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfd)")


def _compile(src: str, extra: list[str], objdir: str) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, *lang, "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if res.stderr.strip():
        # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if any(ln.strip() for ln in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def record_path(lib_path: str) -> str:
    """The build record beside a library: libX.so -> libX.build.json."""
    base = lib_path[:-3] if lib_path.endswith(".so") else lib_path
    return base + ".build.json"


#: tuning variants (built with extra -D flags) live here, one .so each
VARIANTS = os.path.join(PKG, "variants")


def build(extra_flags: list[str] | None = None, verbose: bool = True, out: str = LIB) -> str:
    """Compile and link the library to `out` and record beside it the hash of
    the sources and the extra flags it was built with (fd.library() loads
    the product library only if it was built from the current sources with
    no extra flags).  A build with extra flags (a tuning or instrumented
    variant) compiles into its own object folder."""
    extra = list(extra_flags or [])
    tag = hashlib.sha256(" ".join(extra).encode()).hexdigest()[:8] if extra else ""
    objdir = os.path.join(BUILD, tag) if tag else BUILD
    os.makedirs(objdir, exist_ok=True)
    sources = library_source_hash()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, objdir), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # every kernel stub and symbol must resolve (a host pass that silently
    # drops a kernel stub shows up here, not at the first GPU call)
    import ctypes

    ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    os.replace(tmp, out)
    rec_path = record_path(out)
    with open(rec_path + ".tmp", "w", encoding="utf-8") as f:
        json.dump({"sources_sha256": sources, "flags": extra}, f)
    os.replace(rec_path + ".tmp", rec_path)
    if verbose:
        print(f"built {out}")
    return out


def build_variant(name: str, flags: list[str]) -> str:
    """A tuning variant: the library built with `flags` (build-time knobs,
    -DNAME=value) at variants/<name>.so, for bench.py --library."""
    os.makedirs(VARIANTS, exist_ok=True)
    return build(extra_flags=flags, out=os.path.join(VARIANTS, f"{name}.so"))


if __name__ == "__main__":
    # python -m decode_attention_03_amd.build [NAME -DKNOB=value ...]
    if len(sys.argv) > 2:
        build_variant(sys.argv[1], sys.argv[2:])
    else:
        build()
