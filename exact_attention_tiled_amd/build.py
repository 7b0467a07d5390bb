"""Build step: compile the HIP kernels and the C ABI into lib/libattn.so for gfx950.

    python -m exact_attention_tiled_amd.build [--verbose]

hipcc cross-compiles for gfx950 without a GPU present. Packed-fp32 instruction selection is
switched off for all device code (-packed-fp32-ops); fp32 atomics use the hardware
instructions (-munsafe-fp-atomics; device memory from hipMalloc is coarse-grained). MFMA
results stay in architectural VGPRs (-amdgpu-mfma-vgpr-form): every accumulator is also
read by vector instructions (softmax, rescale), and accumulation registers would cost a
copy each way.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libattn.so")
# Race-exposure build (tests only): every LDS buffer is overwritten with a finite sentinel
# before each refill, so that a missing barrier corrupts results deterministically.
POISON_LIB_PATH = os.path.join(LIB_DIR, "libattn_poison.so")
SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_abi.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libattn.so")
    return path


def compile_command(out: str = LIB_PATH, poison_lds: bool = False) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-munsafe-fp-atomics", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"] + \
        (["-DATTN_DEBUG_POISON_LDS"] if poison_lds else []) + \
        [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out]


def build(verbose: bool = False, poison_lds: bool = False) -> str:
    """Compile every source into lib/libattn.so, or with poison_lds into the race-exposure
    library lib/libattn_poison.so (always recompiles). Returns the path."""
    os.makedirs(LIB_DIR, exist_ok=True)
    path = POISON_LIB_PATH if poison_lds else LIB_PATH
    tmp = path + ".tmp"
    cmd = compile_command(tmp, poison_lds)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, path)
    return path


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
    print(build(verbose="--verbose" in sys.argv, poison_lds=True))
