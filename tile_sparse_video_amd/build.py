"""Builds libvsa.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvsa.so")
SOURCES = ["plan.cpp", "timing.cpp", "groups.cpp", "coarse.hip", "fine.hip", "gemm.hip",
           "backward.hip", "static_ws.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Bit-exact stages (tile means, fused-multiply-add score chains) rely on no
    # implicit contraction and IEEE fp32 division with denormals kept.
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Per-source extras. The fine kernel rescales its O accumulators with VALU
# ops; MFMA accumulators in VGPRs avoid bouncing them through AGPRs. Its
# scores and running maxima are never NaN (padding keys are -inf), so max
# operations need no NaN-quieting canonicalisation. The backward kernels keep
# their long-lived dK/dV and dQ accumulators in AGPRs (the default form), which
# leaves the VGPRs to the operands in flight.
PER_SOURCE = {
    "fine.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless.
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (build(sanitize=True)):
# each flag applies to the host compilation only, never to the gfx950 code.
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]
SANITIZED_LIB = os.path.join(HERE, "_build_san", "libvsa.so")


def build(verbose: bool = False, extra_flags=(), sanitize: bool = False) -> str:
    """Compiles every source and links libvsa.so in-tree. sanitize=True builds the
    host-sanitizer variant into _build_san/libvsa.so instead (load it with
    VSA_LIBRARY=<path> and the clang ASan runtime preloaded; tests/run_sanitized.py
    does both)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build_san" if sanitize else "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    host_san = [x for f in SANITIZE for x in ("-Xarch_host", f)] if sanitize else []
    objs = [os.path.join(objdir, src + ".o") for src in SOURCES]
    cmds = [[hipcc, *HIPCC_FLAGS, *PER_SOURCE.get(src, []), *host_san, *extra_flags, *inc, "-c",
             os.path.join(CSRC, src), "-o", obj] for src, obj in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    lib = SANITIZED_LIB if sanitize else LIB
    link_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-shared-libsan"] if sanitize else []
    tmp = lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_san, *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
