"""Build the HIP libraries in-tree for gfx950 with hipcc.

  bitplane_quantized_expert_amd/libpm.so   the product library (include/pm.h)
  synth/libpmsynth.so                      device filler of the seeded inputs
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
ARCH = os.environ.get("PM_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay off; sums are written with explicit fmaf
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-Wall", "-Wno-unused-function",
]

TARGETS = [
    (os.path.join(PKG, "libpm.so"),
     [os.path.join(PKG, "csrc", "pm_host.cpp"), os.path.join(PKG, "csrc", "pm_cache.cpp"),
      os.path.join(PKG, "csrc", "pm_kernels.hip"), os.path.join(PKG, "csrc", "pm_encoder.hip"),
      os.path.join(PKG, "csrc", "pm_mfma.hip")]),
    (os.path.join(ROOT, "synth", "libpmsynth.so"),
     [os.path.join(ROOT, "synth", "synth_device.hip")]),
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose=False):
    for out, srcs in TARGETS:
        tmp = out + ".tmp"
        cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include")]
        # .cpp sources hold host code only; compile them as HIP so one link works
        for s in srcs:
            cmd += (["-x", "hip", s] if s.endswith(".cpp") else [s])
        cmd += ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
        os.replace(tmp, out)
    return [t for t, _ in TARGETS]


if __name__ == "__main__":
    for p in build(verbose=True):
        print("built", p)
