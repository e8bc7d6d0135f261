"""Builds libsdv.so (the gfx950 verify-step library) and libsdv_probe.so (a
measurement probe that bench.py alone loads) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libsdv.so")
SOURCES = ["sdv_abi.cpp", "attn.hip", "attn_gqa.hip", "attn_mla.hip", "lm_head.hip", "accept.hip", "rollback.hip"]
PROBE_LIB_PATH = os.path.join(HERE, "libsdv_probe.so")
PROBE_SOURCES = ["probe_mfma.hip", "probe_hbm.hip"]
ARCH = "gfx950"

# -Xclang -target-feature -Xclang -packed-fp32-ops keeps the compiler from
# emitting packed fp32 VALU instructions; the host pass warns that it does not
# know the feature, which is harmless.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]

# Per-source extras.  The attention kernels keep many fp32 accumulators and
# resident Q^T fragments per lane (attn_mla.hip: 256 + 144 registers): MFMA
# results in VGPRs (A/B operands may then sit in AGPRs) is the register
# assignment that fits them without spilling to scratch.  The
# attention kernels' LDS DMA sets M0 in inline asm; they have no other M0 use,
# so the reserved-register clobber warning is silenced for them.
EXTRA_FLAGS = {
    "attn_mla.hip": ["-Wno-inline-asm"],
    "attn_gqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-Wno-inline-asm"],
}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    procs = []
    objs = []
    probe_objs = []
    for src in SOURCES + PROBE_SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD_DIR, src + ".o")
        (probe_objs if src in PROBE_SOURCES else objs).append(obj)
        cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
        while sum(p.poll() is None for _, p in procs) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        msg = "\n".join(l for l in (out or "").splitlines()
                        if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            print(msg, file=sys.stderr)
        elif verbose and msg.strip():
            print(msg)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for lib_path, lib_objs in ((LIB_PATH, objs), (PROBE_LIB_PATH, probe_objs)):
        tmp = lib_path + ".tmp"
        cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *lib_objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib_path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
