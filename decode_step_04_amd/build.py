"""Builds libqdec.so (the HIP library) in-tree with hipcc for gfx950.

Every HIP source is compiled with -O3, IEEE fp32 division/sqrt, packed-fp32 instructions
disabled, hidden visibility (only the qdec_* C ABI is exported), then linked into
decode_step_04_amd/libqdec.so.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqdec.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# (source, object, extra flags): gemv.hip is built once per weight type and once for its
# dispatcher, in parallel.  attention.hip and prefill.hip keep matrix-core accumulators in
# ordinary vector registers (in the accumulation registers every rescale of the attention's
# running sums would copy them out and back, and the GEMM tiles would need more registers in
# all); prefill_attn.hip is built without IEEE mode and NaN semantics.
SOURCES = [("gemv.hip", "gemv_f32", ["-DQD_GEMV_PART=0"]),
           ("gemv.hip", "gemv_bf16", ["-DQD_GEMV_PART=1"]),
           ("gemv.hip", "gemv_i8", ["-DQD_GEMV_PART=2"]),
           ("gemv.hip", "gemv_i8g", ["-DQD_GEMV_PART=3"]),
           ("gemv.hip", "gemv_i4g", ["-DQD_GEMV_PART=4", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
           ("gemv.hip", "gemv_dispatch", ["-DQD_GEMV_PART=-1"]),
           ("attention.hip", "attention", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]), ("misc.hip", "misc", []),
           ("prefill.hip", "prefill", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
           ("prefill_attn.hip", "prefill_attn", ["-mno-amdgpu-ieee", "-fno-honor-nans"]),
           ("sample.hip", "sample", []),
           ("runtime.hip", "runtime", [])]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(entry, verbose: bool) -> str:
    src, name, extra = entry
    obj = os.path.join(OUT_DIR, name + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; nothing else is expected
    noise = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0 or (verbose and noise):
        sys.stderr.write("\n".join(noise) + "\n")
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
