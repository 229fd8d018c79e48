"""Build libpa.so (HIP, gfx950) in-tree with hipcc.

    python -m paged_kv_cache_95_amd.build [--jobs N]

Compiles every source under csrc/ to an object file in parallel, then links
paged_kv_cache_95_amd/libpa.so and the debug build paged_kv_cache_95_amd/libpa_debug.so
(the same objects, with the C ABI layer compiled with PA_DEBUG_CHECKS: device-data
contract checks ahead of every kernel call). Always recompiles (this is the build
check).
"""
import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpa.so")
OUT_DEBUG = os.path.join(HERE, "libpa_debug.so")
# the source compiled a second time, with -DPA_DEBUG_CHECKS, for libpa_debug.so
DEBUG_LAYER = "api.cpp"
# sources linked into libpa_debug.so only (the device-data checks and their per-GPU
# state; the release layer never calls them)
DEBUG_ONLY = ("validate.hip",)
BUILD_DIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
# No fast-math: the FP8 quantiser relies on correctly rounded fp32 division.
# Packed fp32 instructions are switched off for all device code.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def compile_one(src, debug=False):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + (".debug.o" if debug else ".o"))
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    flags = ["-DPA_DEBUG_CHECKS=1"] if debug else []
    cmd = [hipcc()] + lang + COMMON + flags + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs=None, verbose=True):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    debug_src = [f for f in srcs if os.path.basename(f) == DEBUG_LAYER]
    jobs = jobs or min(len(srcs) + 1, os.cpu_count() or 4)
    # the slowest sources first, so that the pool is not left waiting on one of them
    order = sorted(srcs, key=lambda f: -os.path.getsize(f))
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = {f: ex.submit(compile_one, f) for f in order}
        dbg = [ex.submit(compile_one, f, True) for f in debug_src]
        objs = [futs[f].result() for f in srcs]
        dbg_objs = [d.result() for d in dbg]
    link([o for f, o in zip(srcs, objs) if os.path.basename(f) not in DEBUG_ONLY], OUT)
    debug_of = dict(zip(debug_src, dbg_objs))
    link([debug_of.get(f, o) for f, o in zip(srcs, objs)], OUT_DEBUG)
    if verbose:
        print(f"built {OUT} and {OUT_DEBUG}", flush=True)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    try:
        build(args.jobs)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
