"""Build libconvrot.so (gfx950) in-tree with hipcc.

    python -m rotation_quantized_int8_amd.build      # or build(verbose=True)

Every HIP source under csrc/ is compiled for gfx950 only.  Floating-point
contraction is off (the W8A8 epilogue's operation order is part of the
contract), packed fp32 instructions are disabled, and MFMA accumulators are
kept in VGPRs.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libconvrot.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: with AGPR accumulators the register
    # allocator copies them AGPR<->VGPR around the pipelined loop's transitions
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libconvrot)")
    return exe


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every csrc/*.hip and link LIB_PATH; returns the library path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="convrot_build_") as tmp:
        objs, procs = [], []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0), verbose)
        for pr in procs:
            _wait(pr, verbose)
        tmp_lib = os.path.join(tmp, LIB_NAME)
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        if verbose:
            print(" ".join(link), flush=True)
        r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}")
        shutil.move(tmp_lib, LIB_PATH)
    return LIB_PATH


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # hipcc's host pass does not know the packed-fp32 target feature; drop that noise
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l]
    if p.returncode != 0:
        raise RuntimeError(f"compile failed for {src}:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
