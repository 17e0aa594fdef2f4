"""Build libw4.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every source is compiled for gfx950 only, with packed fp32 instructions disabled and without
fast-math: fp32 division stays correctly rounded, which the bit-exact codec kernels rely on.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libw4.so")
SOURCES = ["abi.hip", "codec.hip", "decode.hip", "decode_i8.hip", "decode_mfma.hip",
           "decode_stream.hip", "gemm.hip", "gemm_w4a8.hip", "qat_repack.hip",
           "gptq.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=fast",
]
# Per-source additions.  The GEMM keeps its MFMA accumulators in ordinary VGPRs: with the default
# heuristics the register allocator rotates them through AGPRs and spends about one move per
# MFMA inside the main loop.
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def assembly(src: str, out: str) -> None:
    """Write the gfx950 assembly of one source (for inspecting the generated ISA)."""
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
