"""Build libmoe.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m mixture_experts_layer_router_amd.build

Every .hip file under csrc/ is compiled to an object in _build/ and linked into
mixture_experts_layer_router_amd/_lib/libmoe.so.  Packed-fp32 VALU instructions
are disabled for all device code.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


# Per-file extra flags.  decode.hip: its atomics are all issued by one lane,
# so the wave-level atomic combiner only adds an immediate wait on each result.
# gemm.hip: its direct-to-LDS loads are inline asm that sets M0 (a reserved
# register nothing else in that file uses); silence the clobber warning.  Its
# matrix instructions write VGPRs: the FP8 b128 promotion then reads the
# block products with plain FMAs instead of copying each out of an AGPR, and
# the operand registers go to the AGPRs (measured: routed gate/up 879 -> 826
# us, down 532 -> 505 us at 4,096 tokens).
# gemm2.hip: its 288 accumulator registers per lane (256 main + 32 for the
# extra row block) exceed the 256 AGPRs; with matrix results in VGPRs the
# compiler splits the accumulators over both files and keeps the operands in
# AGPRs, where the AGPR form shuttled three blocks through a spare AGPR
# range with copies and wait states around every use (2,048-token layer
# 822 -> 754 us).
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
         "gemm.hip": ["-Wno-inline-asm", "-mllvm", "-amdgpu-mfma-vgpr-form"],
         "gemm2.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for obj, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
