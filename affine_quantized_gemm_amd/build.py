"""Build libqmm.so (HIP, gfx950) in-tree with hipcc.

Every translation unit under ``csrc/`` is compiled to an object in
``_build/`` (in parallel) and linked into ``libqmm.so`` next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqmm.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU ops anywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def digest_inputs(root: str = ROOT):
    """Every file the library is compiled from: csrc/*.hip, csrc/*.hpp and
    include/*.h, as (path relative to root, absolute path), sorted."""
    out = []
    for d, exts in ((os.path.join(root, "affine_quantized_gemm_amd", "csrc"), (".hip", ".hpp")),
                    (os.path.join(root, "include"), (".h",))):
        for f in sorted(os.listdir(d)):
            if f.endswith(exts):
                p = os.path.join(d, f)
                out.append((os.path.relpath(p, root).replace(os.sep, "/"), p))
    return out


def source_digest(root: str = ROOT) -> str:
    """SHA-256 (first 16 hex digits) over the names and contents of
    :func:`digest_inputs`; compiled into the library as qmm_build_digest()."""
    h = hashlib.sha256()
    for rel, p in digest_inputs(root):
        with open(p, "rb") as f:
            data = f.read()
        h.update(rel.encode() + b"\0" + str(len(data)).encode() + b"\0" + data)
    return h.hexdigest()[:16]


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *COMMON, f'-DQMM_SOURCE_DIGEST="{digest}"', "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name; that note is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libqmm.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    digest = source_digest()
    # the largest translation units first, so that they do not start last
    order = sorted(srcs, key=lambda f: -os.path.getsize(f))
    with cf.ThreadPoolExecutor(max_workers=min(os.cpu_count() or 8, 16, len(srcs))) as ex:
        done = dict(zip(order, ex.map(lambda src: _compile(src, digest), order)))
    objs = [done[f] for f in srcs]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources (source digest {digest})")
    return LIB


if __name__ == "__main__":
    build()
