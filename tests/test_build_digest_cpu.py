"""The library records the digest of the sources it was built from, and the
binding refuses a library whose sources have changed since (a stale binary
would otherwise run silently on the GPU in place of the code under test)."""

import os
import shutil
import subprocess
import sys

from conftest import ROOT

import affine_quantized_gemm_amd as Q
from affine_quantized_gemm_amd import build as B


def test_loaded_library_matches_its_sources():
    assert Q.BUILD_DIGEST == B.source_digest()
    assert len(Q.BUILD_DIGEST) == 16
    names = [rel for rel, _ in B.digest_inputs()]
    assert "include/qmm.h" in names and "affine_quantized_gemm_amd/csrc/qmm_mfma_reg.hpp" in names


def _copy_tree(dst):
    shutil.copytree(os.path.join(ROOT, "include"), os.path.join(dst, "include"))
    pkg = os.path.join(dst, "affine_quantized_gemm_amd")
    shutil.copytree(os.path.join(ROOT, "affine_quantized_gemm_amd"), pkg,
                    ignore=shutil.ignore_patterns("_build", "__pycache__"))
    return pkg


def _import_in(root):
    env = dict(os.environ, PYTHONPATH=root)
    return subprocess.run([sys.executable, "-c", "import affine_quantized_gemm_amd as Q; print(Q.BUILD_DIGEST)"],
                          cwd=root, env=env, capture_output=True, text=True, timeout=300)


def test_changed_source_makes_the_library_stale(tmp_path):
    root = str(tmp_path)
    pkg = _copy_tree(root)
    r = _import_in(root)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == Q.BUILD_DIGEST
    # one changed line in one kernel source: the same binary is now refused
    src = os.path.join(pkg, "csrc", "qmm_mfma_reg.hpp")
    with open(src, "a") as f:
        f.write("// changed\n")
    assert B.source_digest(root) != Q.BUILD_DIGEST
    r = _import_in(root)
    assert r.returncode != 0
    assert "StaleLibraryError" in r.stderr and "rebuild" in r.stderr
