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
SOURCES = ["abi.hip", "codec.hip", "decode.hip", "decode_i8.hip", "decode_mfma.hip", "decode_split.hip",
           "decode_stream.hip", "decode_w4a8_mfma.hip", "gemm.hip", "gemm_w4a8.hip", "qat_repack.hip",
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


# The test library: the same sources, with the kernel-choice hook of decode_i8.hip compiled in
# (W4_TEST_HOOKS). Only the tests load it; the product library has no such entry point.
HOOKS_LIB = os.path.join(HERE, "libw4_hooks.so")
HOOKED = {"decode_i8.hip"}


def _compile(src: str, verbose: bool, hooks: bool = False) -> str:
    stem = os.path.splitext(src)[0] + ("_hooks" if hooks else "")
    obj = os.path.join(BUILD, stem + ".o")
    defs = ["-DW4_TEST_HOOKS"] if hooks else []
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [(s, True) for s in sorted(HOOKED)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    plain = objs[:len(SOURCES)]
    hooked = {s: o for (s, h), o in zip(jobs, objs) if h}
    _link(plain, LIB, verbose)
    _link([hooked.get(s, o) for s, o in zip(SOURCES, plain)], HOOKS_LIB, verbose)
    return LIB


def assembly(src: str, out: str) -> None:
    """Write the gfx950 assembly of one source (for inspecting the generated ISA)."""
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
