"""Build libdcnv4.so (HIP, gfx950) in-tree with hipcc.

    python -m deformable_convolution_vision_dcnv4_amd.build [--asm DIR]

Flags: contraction off (the binary32 operation order is part of the
operator's contract), packed-fp32 instructions disabled, -O3.
"""
import argparse
import concurrent.futures
import glob
import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdcnv4.so")
ARCH = "gfx950"

HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
             "-ffp-contract=off", "-fno-gpu-rdc",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def source_hash(scope="all"):
    """Short digest of the kernel sources and the public headers: names a
    build, so that counter measurements can be matched to the code they
    were taken on.  scope="forward": only the files the forward operator's
    kernels are built from (not the module's or the backward's), so that a
    change elsewhere keeps the forward's counter records valid."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*"))) + sorted(glob.glob(os.path.join(INCLUDE, "*.h")))
    for path in files:
        if not os.path.isfile(path) or path.endswith((".so", ".tmp")):
            continue
        if scope == "forward" and any(w in os.path.basename(path) for w in ("module", "backward")):
            continue
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + b"\0" + fh.read())
    h.update(" ".join(HIP_FLAGS).encode())
    return h.hexdigest()[:16]


def hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(verbose=False, asm_dir=None, jobs=None):
    """Compile every source to an object in parallel (one hipcc per file),
    then link the shared library."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(src).replace(".hip", ".o")) for src in sources()]
    cmds = [[hipcc()] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, src]
            for src, obj in zip(sources(), objs)]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for cmd, r in zip(cmds, ex.map(lambda c: subprocess.run(c, cwd=CSRC, capture_output=True, text=True),
                                       cmds)):
            if verbose:
                print(" ".join(cmd), flush=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{r.stderr}")
    link = [hipcc()] + HIP_FLAGS + ["-shared", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True, cwd=CSRC)
    os.replace(LIB + ".tmp", LIB)
    if asm_dir:
        # device ISA of each source, for inspection
        os.makedirs(asm_dir, exist_ok=True)
        for src in sources():
            out = os.path.join(asm_dir, os.path.basename(src).replace(".hip", ".s"))
            subprocess.run([hipcc()] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC, "--cuda-device-only",
                                                    "-S", "-o", out, src], check=True, cwd=CSRC)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="keep intermediate files (ISA) in this directory")
    args = ap.parse_args()
    print(build(verbose=True, asm_dir=args.asm))
