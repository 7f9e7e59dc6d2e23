"""Build libdflash.so (the HIP library behind include/dflash.h) in-tree for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["api.hip", "kernels_weights.hip", "kernels_step.hip", "kernels_chain.hip"]
LIB = os.path.join(PKG, "libdflash.so")
ARCH = os.environ.get("DFLASH_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms are kept out of the generated code; the host pass warns
# that it does not know the feature, which is harmless.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        cmd = [hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile of {src} failed:\n{r.stdout}\n{r.stderr}")
        if verbose:
            print(" ".join(cmd))
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, *FLAGS, "-shared", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def resource_usage(sources=SOURCES) -> dict:
    """Per-kernel register, scratch and occupancy figures the compiler reports for gfx950.

    Compiles the device side of each source once more (nothing is written) and
    parses the kernel-resource-usage remarks: {kernel: {"vgprs", "agprs",
    "sgprs", "scratch", "occupancy"}}.
    """
    hipcc = _hipcc()
    keys = {"VGPRs": "vgprs", "AGPRs": "agprs", "TotalSGPRs": "sgprs",
            "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy"}

    def one(src: str) -> dict:
        cmd = [hipcc, *FLAGS, "--cuda-device-only", "-c", os.path.join(CSRC, src), "-o", os.devnull,
               "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile of {src} failed:\n{r.stderr}")
        out, cur = {}, None
        for line in r.stderr.splitlines():
            if "remark:" not in line:
                continue
            text = line.split("remark:", 1)[1].split(" [-Rpass", 1)[0].strip()
            name, _, val = text.rpartition(": ")
            if name == "Function Name":
                cur = out.setdefault(val, {})
            elif cur is not None and name in keys:
                cur[keys[name]] = int(val)
        return out

    res = {}
    with ThreadPoolExecutor(len(sources)) as ex:
        for part in ex.map(one, sources):
            res.update(part)
    return res


if __name__ == "__main__":
    print(build(verbose=True))
