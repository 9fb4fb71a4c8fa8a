"""Build of the gfx950 HIP library (libss.so) in-tree with hipcc.

Every HIP translation unit is compiled for gfx950 only, with packed-fp32 code
generation turned off, and linked into selective_state_space_34_amd/lib/libss.so.
"""
import concurrent.futures as cf
import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libss.so")

SOURCES = ["ss_api.cpp", "ss_fwd.hip", "ss_fwdg.hip", "ss_carry.hip", "ss_bwd.hip", "ss_step.hip",
           "ss_block.hip"]
HEADERS = ["ss_device.h", "ss_kernels.h", "ss_plan.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# code-generation flags (part of the build identity); include paths are added per build
CODEGEN = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]
FLAGS = CODEGEN + [f"-I{INCLUDE}", f"-I{CSRC}"]


def tree_id(csrc: str = CSRC, include: str = INCLUDE) -> str:
    """Identity of the sources the library is built from: SHA-256 over every file of csrc/
    (name and bytes, sorted by name), include/ss.h and the code-generation flags.  build()
    bakes it into libss.so (ss_build_id); load() refuses a library whose identity differs."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        p = os.path.join(csrc, f)
        if f.startswith(".") or not os.path.isfile(p):
            continue
        h.update(f.encode() + b"\0")
        with open(p, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    with open(os.path.join(include, "ss.h"), "rb") as fh:
        h.update(fh.read())
    h.update(" ".join(CODEGEN).encode())
    return h.hexdigest()


def _compile(src, ident):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, f'-DSS_BUILD_ID="{ident}"', "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def stale() -> bool:
    """True when libss.so is missing or was built from other sources than the tree's."""
    if not os.path.exists(LIB):
        return True
    with open(LIB, "rb") as fh:
        return tree_id().encode() not in fh.read()


def build(jobs: int = 4) -> str:
    """Compile every translation unit for gfx950 and link libss.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    ident = tree_id()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, ident), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
