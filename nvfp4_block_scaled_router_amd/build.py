"""Build libnvfp4moe.so: the HIP kernels for gfx950 and the C ABI, in-tree.

Every source compiles with hipcc for gfx950 only. Packed-FP32 VALU instructions
are disabled (-packed-fp32-ops) for all device code; the quantiser is compiled
without floating-point contraction and with correctly rounded fp32 division so
that its bytes are a pure function of its input bits.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4moe.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-Wno-unused-command-line-argument"]
SOURCES = {
    "api.cpp": [],
    "route.hip": [],
    "quant.hip": ["-ffp-contract=off"],
    "pack.hip": [],
    # MFMA accumulators in architectural VGPRs: the default AGPR form makes the register
    # allocator shuttle accumulators between the two files inside the K loops
    # (v_accvgpr_read/write, about one per MFMA) and raises the register count.
    "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD_DIR, src.replace(".", "_") + ".o")
        objs.append(obj)
        cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only feature flag; that note is harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode):
            print(f"--- {src}\n" + "\n".join(lines), file=sys.stderr, flush=True)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
