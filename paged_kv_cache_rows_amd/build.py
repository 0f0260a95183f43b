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


RESOURCE_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes",
                   "Occupancy [waves/SIMD]": "waves_per_simd", "SGPRs Spill": "sgpr_spill",
                   "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds_bytes"}
RECORD_JSON = os.path.join(ROOT, "profiles", "kernel_resources.json")
RECORD_MD = os.path.join(ROOT, "profiles", "kernel_resources.md")


def parse_resources(path: str = os.path.join(BUILD, "resource_usage.txt")) -> dict:
    """Per-kernel resource records from the compiler's kernel-resource-usage remarks of the last
    build: {demangled name: {sgprs, vgprs, agprs, scratch_bytes, waves_per_simd, sgpr_spill,
    vgpr_spill, lds_bytes}}."""
    recs, cur = {}, None
    with open(path) as f:
        for ln in f:
            if "remark:" not in ln:
                continue
            body = ln.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
            key, _, val = body.partition(":")
            key, val = key.strip(), val.strip()
            if key == "Function Name":
                cur = val
                recs[cur] = {}
            elif cur is not None and key in RESOURCE_FIELDS:
                recs[cur][RESOURCE_FIELDS[key]] = int(val)
    names = list(recs)
    p = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    demangled = p.stdout.splitlines() if p.returncode == 0 and len(p.stdout.splitlines()) == len(names) else names
    return {d: recs[n] for n, d in zip(names, demangled)}


def write_record():
    """Write the current build's per-kernel resources to profiles/ (JSON and a Markdown table)."""
    import json
    recs = parse_resources()
    with open(RECORD_JSON, "w") as f:
        json.dump(recs, f, indent=1, sort_keys=True)
        f.write("\n")
    cols = ["vgprs", "agprs", "sgprs", "scratch_bytes", "vgpr_spill", "sgpr_spill", "lds_bytes", "waves_per_simd"]
    lines = ["# Kernel resources (gfx950, hipcc of ROCm 7.2, -O3)", "",
             "Written by `python -m paged_kv_cache_rows_amd.build --record` from the compiler's",
             "kernel-resource-usage remarks of the build (`_build/resource_usage.txt`); "
             "`tests/test_kernel_resources.py` fails",
             "when a kernel spills or when the build no longer matches this record.", "",
             "| kernel | " + " | ".join(cols) + " |", "|---|" + "---:|" * len(cols)]
    for name in sorted(recs):
        r = recs[name]
        lines.append(f"| `{name}` | " + " | ".join(str(r.get(c, "")) for c in cols) + " |")
    with open(RECORD_MD, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
    if "--record" in sys.argv:
        write_record()
