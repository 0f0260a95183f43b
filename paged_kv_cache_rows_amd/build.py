"""Build libkvpaged.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc.

    python -m paged_kv_cache_rows_amd.build [--verbose]

Every call recompiles.  Objects go to paged_kv_cache_rows_amd/_build/, the library to
paged_kv_cache_rows_amd/libkvpaged.so, and the compiler's per-kernel resource report
(VGPR/AGPR/SGPR counts, spills, LDS bytes, occupancy) to _build/resource_usage.txt.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvpaged.so")
# the benchmark's HBM read probe, a library of its own (not part of the attention ABI)
PROBE_LIB = os.path.join(HERE, "libkvprobe.so")
PROBE_SOURCES = ["probe.hip"]

SOURCES = ["api.cpp", "kernels_io.hip", "kernels_valu.hip", "kernels_mfma.hip", "scratch.hip"]
ARCH = "gfx950"
# Packed fp32 instructions are turned off for every HIP translation unit.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


# Per-source flags.  The MFMA kernels keep their accumulators in ordinary VGPRs (gfx950 MFMA
# reads and writes them directly); with AGPR accumulators the softmax and the rescale of the
# output move every value through v_accvgpr_read/write.
SOURCE_FLAGS = {
    "kernels_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: str, verbose: bool):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"]
    cmd += SOURCE_FLAGS.get(src, [])
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{p.stdout}\n{p.stderr}")
    report = [ln for ln in p.stderr.splitlines() if "remark:" in ln]
    return obj, report


def _link(objs, lib: str, verbose: bool):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        results = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        for src in SOURCES:
            rep = results[src][1]
            f.write("\n".join(rep) + ("\n" if rep else ""))
    _link([results[s][0] for s in SOURCES], LIB, verbose)
    _link([results[s][0] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
