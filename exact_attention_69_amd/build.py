"""Build libexattn.so (HIP kernels for gfx950 + the C-ABI entry points).

Usage: ``python -m exact_attention_69_amd.build [-j N] [--verbose] [--no-poison] [--sanitize]``.
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file, where the Python binding loads it from, and so is
its LDS-poisoning debug twin, libexattn_poison.so.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG_DIR, "libexattn.so")
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def common_flags():
    return [
        "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function",
        # no packed fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


# Flags for single sources: some instantiations are compiled with LLVM's
# max-ilp machine scheduler, where it measured faster (the d = 128 backward
# without a mask; the d = 128 forward without a mask and the d = 256 forward
# with a window); each unit's header gives the measurements.
MAX_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
SOURCE_FLAGS = {"bwd_bf16_d128.hip": MAX_ILP, "fwd_bf16_ilp.hip": MAX_ILP}


def sources():
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".hip") or name.endswith(".cpp"):
            out.append(os.path.join(CSRC, name))
    return out


def _compile(src, verbose, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    unit_flags = SOURCE_FLAGS.get(os.path.basename(src), [])
    cmd = [hipcc()] + common_flags() + unit_flags + list(extra) + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return obj


def build(jobs=None, verbose=False, build_dir=BUILD, lib=LIB, extra=()):
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, lib)
    return lib


# Debug build whose kernels fill their LDS with NaN bytes before first use
# (EXATTN_POISON_LDS, device_common.hpp): run against the ordinary build, any
# read of LDS that the kernel did not write first shows up as a difference.
# It sits next to the ordinary library so that it travels with the package.
POISON_LIB = os.path.join(PKG_DIR, "libexattn_poison.so")


def build_poisoned(jobs=None, verbose=False):
    return build(jobs, verbose, os.path.join(BUILD, "poison"), POISON_LIB, ["-DEXATTN_POISON_LDS"])


# Host sanitizers for the C-ABI code (argument validation, size arithmetic,
# workspace offsets): each -fsanitize= applies to the host compilation only.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(BUILD, "san", "libexattn_san.so")


def asan_runtime():
    """Path of clang's shared AddressSanitizer runtime (to preload into the
    Python process that loads the sanitizer build), or None."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_sanitized(verbose=False):
    """libexattn_san.so: the C-ABI entry points (api.cpp) compiled with host
    AddressSanitizer and UndefinedBehaviorSanitizer, linked with the kernels'
    ordinary objects.  For host-only tests of the validation paths (load it
    with EXATTN_LIBRARY set and the runtime from asan_runtime() preloaded)."""
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    objs = []
    for src in sources():
        if os.path.basename(src) == "api.cpp":
            obj = os.path.join(os.path.dirname(SAN_LIB), "api.cpp.o")
            cmd = [hipcc(), "-x", "hip"] + common_flags() + ["-g", "-O1"] + SAN_FLAGS + ["-c", src, "-o", obj]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
            objs.append(obj)
        else:
            obj = os.path.join(BUILD, os.path.basename(src) + ".o")
            # sources include each other: rebuild when any of them is newer
            newest = max(os.path.getmtime(os.path.join(CSRC, f)) for f in os.listdir(CSRC))
            if not os.path.exists(obj) or os.path.getmtime(obj) < newest:
                obj = _compile(src, verbose)
            objs.append(obj)
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", SAN_LIB] + objs + SAN_FLAGS[:4] + \
        ["-shared-libsan"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return SAN_LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("-j", "--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="also build the host-sanitizer library of the C-ABI code (_build/san/)")
    ap.add_argument("--no-poison", action="store_true",
                    help="skip the LDS-poisoning debug library (libexattn_poison.so)")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))
    if not args.no_poison:
        print(build_poisoned(args.jobs, args.verbose))
    if args.sanitize:
        print(build_sanitized(args.verbose))


if __name__ == "__main__":
    sys.exit(main())
