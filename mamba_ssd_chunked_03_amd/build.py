"""Build libssd.so (the HIP library behind include/ssd.h) in-tree for gfx950.

Each translation unit is compiled by hipcc to an object under _build/, in parallel, and
the objects are linked into mamba_ssd_chunked_03_amd/libssd.so.  Always recompiles.

    python -m mamba_ssd_chunked_03_amd.build
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libssd.so")
ARCH = "gfx950"

SOURCES = ["ssd_api.hip", "chunk_cumsum.hip", "state_passing.hip", "chunk_valu.hip",
           "chunk_mfma.hip", "chunk_scan_mfma.hip", "decode_step.hip", "chunk_bwd_valu.hip",
           "chunk_bwd_mfma.hip", "block.hip", "varlen.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=fast",
    # packed fp32 (v_pk_*_f32) stays off: only plain fp32 VALU instructions are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(LIBRARY, file=sys.stderr)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
