"""Builds libmoe_fp8.so (the layer) and synth/libsynth.so (the input generator)
in-tree with hipcc for gfx950."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")

LIB = os.path.join(PKG, "libmoe_fp8.so")
SYNTH_LIB = os.path.join(ROOT, "synth", "libsynth.so")

SOURCES = ["common.hip", "quant.hip", "route.hip", "permute.hip", "gemm_fp8.hip", "combine.hip",
           "backward.hip", "probe.hip", "layer.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # float division and sqrt correctly rounded (448 / amax must be exact)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # MFMA results in VGPRs: the per-block scale FMA reads them directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed for {cmd[-1]}")
    return res


def _compile(src, obj, extra=()):
    _run([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj])
    return obj


def build(jobs=8, save_temps=False):
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-save-temps=obj"] if save_temps else []
    objs = []
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s),
                          os.path.join(BUILD, s.replace(".hip", ".o")), extra)
                for s in SOURCES]
        fs = ex.submit(_compile, os.path.join(ROOT, "synth", "synth.hip"),
                       os.path.join(BUILD, "synth.o"), extra)
        objs = [f.result() for f in futs]
        synth_obj = fs.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", synth_obj, "-o", tmp])
    os.replace(tmp, SYNTH_LIB)
    return LIB


if __name__ == "__main__":
    build(save_temps="--save-temps" in sys.argv)
    print(LIB)
