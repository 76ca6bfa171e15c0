"""Build ``libsp_csr.so`` in-tree from ``csrc/*.hip`` with hipcc for gfx950,
and ``libsp_probes.so`` (the measured-ceiling probes) from ``probes/*.hip``.

Run ``python -m unstructured_sparse_linear_csr_amd.build``.  Every call
recompiles; sources compile in parallel into ``_build/`` and are linked into
the two libraries in ``unstructured_sparse_linear_csr_amd/``.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsp_csr.so")
PROBES = os.path.join(PKG, "probes")
PROBE_LIB = os.path.join(PKG, "libsp_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-FP32 instructions are switched off for all device code: the compiler
# must not form v_pk_* FP32 ops from scalar or float2 code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    noise = "is not a recognized feature for this target"
    rest = "\n".join(l for l in r.stderr.splitlines() if noise not in l).strip()
    if rest:
        sys.stderr.write(rest + "\n")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probes = sorted(glob.glob(os.path.join(PROBES, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(sources) + len(probes))) as ex:
        objs = list(ex.map(_compile, sources + probes))
    _link(objs[:len(sources)], LIB, verbose)
    _link(objs[len(sources):], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
