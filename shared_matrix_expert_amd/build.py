"""Build libedge_moe.so (HIP, gfx950) in-tree with hipcc.

    python -m shared_matrix_expert_amd.build

Each source under csrc/ compiles to an object in _build/ (in parallel), then
one shared library is linked next to this file.  Packed-FP32 instruction
selection is switched off for the device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libedge_moe.so")
SOURCES = ["api.hip", "router.hip", "dispatch.hip", "gemm.hip", "decode.hip", "layer.hip",
           "prefill.hip", "calib.hip", "mx.hip", "prefetch.hip", "cache.hip"]
ARCH = "gfx950"


# The source file of each kernel family (by kernel-name prefix); a stored
# profile of a kernel stays valid while that file and the headers it includes are
# unchanged.
KERNEL_SOURCES = (("dec_layer", "layer.hip"), ("pl_", "layer.hip"), ("dec_", "decode.hip"),
                  ("router_", "router.hip"), ("perm_", "dispatch.hip"), ("pf_", "prefill.hip"),
                  ("mfma_peak", "calib.hip"), ("mx_", "mx.hip"), ("prefetch_", "prefetch.hip"), ("cache_", "cache.hip"),
                  ("copy_bytes", "gemm.hip"))


def include_closure(src: str, root_csrc: str = CSRC, root_inc: str = os.path.join(ROOT, "include"),
                    read=None) -> list:
    """Files `src` (under csrc/) compiles from: itself and every header it
    includes with #include "..." (internal headers and the public header),
    transitively; sorted by path, the source last.  `read(path)` returns a file's text
    (default: the working tree)."""
    read = read or (lambda path: open(path, encoding="utf-8").read())
    seen, todo = set(), [os.path.join(root_csrc, src)]
    while todo:
        path = todo.pop()
        if path in seen:
            continue
        seen.add(path)
        for line in read(path).splitlines():
            t = line.strip()
            if t.startswith("#include") and '"' in t:
                name = t.split('"')[1]
                for base in (root_csrc, root_inc):
                    cand = os.path.join(base, name)
                    try:
                        read(cand)
                    except (OSError, KeyError):
                        continue
                    todo.append(cand)
                    break
    src_path = os.path.join(root_csrc, src)
    return sorted(p for p in seen if p != src_path) + [src_path]


def sources_digest(kernel: str = "", read=None) -> str:
    """sha256 identifying the code a stored profile was taken from: with a
    kernel, the kernel's source file and the headers it includes (so that an
    edit elsewhere leaves its profiles valid); without one, every source and
    header and the public header."""
    import hashlib
    read_b = (lambda path: open(path, "rb").read()) if read is None else (lambda path: read(path).encode())
    h = hashlib.sha256()
    hit = [f for pre, f in KERNEL_SOURCES if kernel.startswith(pre)] if kernel else []
    if hit:
        files = include_closure(hit[0], read=read)
    else:
        headers = sorted(f for f in os.listdir(CSRC) if f.endswith(".h"))
        srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
        files = [os.path.join(CSRC, f) for f in headers + srcs] + [os.path.join(ROOT, "include", "edge_moe.h")]
    for path in files:
        h.update(os.path.basename(path).encode() + b"\0" + read_b(path))
    return h.hexdigest()


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


# Per-source code-generation options: the prefill GEMMs keep their MFMA
# results in ordinary VGPRs (the scaled chunk sums are added by VALU FMAs).
EXTRA = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *_flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
