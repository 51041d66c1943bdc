"""Build libg4attn.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m attention_g4attn_amd.build

Each source is compiled by hipcc for gfx950 in parallel, then linked into
attention_g4attn_amd/libg4attn.so.  Packed fp32 instructions are disabled for
all device code.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libg4attn.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "prefill_kv512.hip", "prefill_d256.hip", "prefill_sep512.hip", "prefill_vis.hip",
           "decode_bf16.hip", "decode_fp8.hip", "attn_f32.hip", "cache_fill.hip",
           "decode_noalloc.hip", "decode_mc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}", flush=True)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
