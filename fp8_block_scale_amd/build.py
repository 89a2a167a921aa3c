"""Build libmoe_fp8.so for gfx950 from the HIP sources in csrc/.

Every translation unit is compiled with hipcc (in parallel) and linked into
one shared library next to this file.  Packed FP32 instructions are disabled
for device code, denormals are preserved and no fast-math is used, so IEEE
division and rounding hold where the quantisers need them.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libmoe_fp8.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["plan.hip", "quant.hip", "gateup.hip", "gateup_pipe.hip", "down.hip", "down_pipe.hip", "down_cols.hip",
           "gateup_slices.hip", "fused.hip", "capi.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe_fp8)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=fast",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    ]


def build(verbose=False, jobs=None):
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = compile_flags()

    def one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            msgs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
            if msgs:
                print("\n".join(msgs), file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs or min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
