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

COMPILE_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay off; sums are written with explicit fmaf
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-Wall", "-Wno-unused-function",
]

TARGETS = [
    (os.path.join(PKG, "libpm.so"),
     [os.path.join(PKG, "csrc", "pm_host.cpp"), os.path.join(PKG, "csrc", "pm_cache.cpp"),
      os.path.join(PKG, "csrc", "pm_kernels.hip"), os.path.join(PKG, "csrc", "pm_lut.hip"),
      os.path.join(PKG, "csrc", "pm_encoder.hip"),
      os.path.join(PKG, "csrc", "pm_mfma.hip")]),
    (os.path.join(ROOT, "synth", "libpmsynth.so"),
     [os.path.join(ROOT, "synth", "synth_device.hip")]),
]

# Per-source extra flags.  The LUT kernels issue many independent table
# lookups per step; the machine scheduler's ILP strategy keeps them in flight
# instead of interleaving each with its use.  (The same strategy makes the
# direct kernels about twice as slow, so they stay in another source.)
EXTRA = {
    "pm_lut.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _run(cmd, what, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {what}")


def build(verbose=False, extra_flags=(), out_override=None, only_pm=False):
    """Compile every source to an object (with its own extra flags), then
    link each library.  extra_flags / out_override / only_pm serve tuning and
    profiling builds of libpm."""
    import concurrent.futures as cf
    outs = []
    for out, srcs in (TARGETS[:1] if only_pm else TARGETS):
        if out_override and out.endswith("libpm.so"):
            out = out_override
        objs, jobs = [], []
        for s in srcs:
            obj = os.path.join(os.path.dirname(out), "_build",
                               os.path.basename(s) + "." + os.path.basename(out) + ".o")
            os.makedirs(os.path.dirname(obj), exist_ok=True)
            cmd = [hipcc()] + COMPILE_FLAGS + list(extra_flags) + EXTRA.get(os.path.basename(s), []) + [
                "-I", os.path.join(ROOT, "include"), "-c"]
            # .cpp sources hold host code only; compile them as HIP so one link works
            cmd += (["-x", "hip", s] if s.endswith(".cpp") else [s])
            cmd += ["-o", obj]
            objs.append(obj)
            jobs.append((cmd, os.path.basename(s)))
        with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            list(ex.map(lambda j: _run(j[0], j[1], verbose), jobs))
        tmp = out + ".tmp"
        _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp],
             os.path.basename(out), verbose)
        os.replace(tmp, out)
        outs.append(out)
    return outs


# libpm with its host code under AddressSanitizer and UndefinedBehaviorSanitizer
# (the device code is built as usual): for the host-only tests (the host-backed
# store, the expert caches, routing, the allocator, argument validation), run
# in a process that preloads the ASan runtime.  Every -fsanitize goes to the
# host pass only.
ASAN_LIB = os.path.join(PKG, "libpm_asan.so")
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime():
    """The ASan runtime of the compiler that builds ASAN_LIB (None if absent)."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib",
                                         "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build_sanitized(verbose=False):
    import concurrent.futures as cf
    srcs = TARGETS[0][1]
    flags = [f for f in COMPILE_FLAGS if f != "-O3"] + ["-O1", "-g"] + SANITIZE
    objs, jobs = [], []
    for s in srcs:
        obj = os.path.join(PKG, "_build", os.path.basename(s) + ".asan.o")
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        cmd = [hipcc()] + flags + ["-I", os.path.join(ROOT, "include"), "-c"]
        cmd += (["-x", "hip", s] if s.endswith(".cpp") else [s])
        cmd += ["-o", obj]
        objs.append(obj)
        jobs.append((cmd, os.path.basename(s)))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _run(j[0], j[1], verbose), jobs))
    tmp = ASAN_LIB + ".tmp"
    _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}"] + SANITIZE[:4] +
         ["-shared-libsan"] + objs + ["-o", tmp], os.path.basename(ASAN_LIB), verbose)
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


# libpm with per-workgroup timeline stamps in the LUT kernels (PM_LUT_STAMPS):
# a profiling build for bench.py --wg-timeline, never the product.
STAMPS_LIB = os.path.join(PKG, "libpm_stamps.so")


def build_stamps(verbose=False):
    return build(verbose, extra_flags=["-DPM_LUT_STAMPS"], out_override=STAMPS_LIB, only_pm=True)[0]


if __name__ == "__main__":
    for p in build(verbose=True):
        print("built", p)
    print("built", build_sanitized(verbose=True))
    print("built", build_stamps(verbose=True))
