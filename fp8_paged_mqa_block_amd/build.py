"""Compile the gfx950 HIP kernels and the C-ABI host layer into libpmqa.so (in-tree).

Run as ``python -m fp8_paged_mqa_block_amd.build``.  hipcc cross-compiles for
gfx950 without a GPU present.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = ["pmqa_host.hip", "logits_gfx950.hip", "topk_gfx950.hip", "check_gfx950.hip",
           "kcache_gfx950.hip"]
LIB = os.path.join(PKG, "libpmqa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",  # only the C ABI (PMQA_API) is exported
    # packed fp32 VALU forms stay off: the compiler may not form v_pk_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels' leading scalar arguments (context lengths, batch, bounds,
    # the tables and q to warm) are preloaded into SGPRs by the dispatch, so a
    # wave's first loads need not wait for the argument block
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(PKG, "csrc", s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise and verbose:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
