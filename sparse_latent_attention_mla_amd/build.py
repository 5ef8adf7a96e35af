"""Build the gfx950 HIP library libmla.so in-tree with hipcc.

Every translation unit is compiled for gfx950 only, without packed-fp32
instructions (-packed-fp32-ops), with IEEE fp32 division and square root, and
linked into sparse_latent_attention_mla_amd/libmla.so.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "mla")
LIB = os.path.join(HERE, "libmla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.cpp", "profile.cpp", "options.cpp", "append.hip", "indexer.hip", "topk.hip", "pool.hip", "decode.hip", "compress.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-source extras: MFMA results in ordinary VGPRs, so accumulators are never
# copied between accumulation and vector registers (decode: the output tile in
# the chunk loop; indexer: the scores of every tile before ReLU).
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src, verbose):
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
