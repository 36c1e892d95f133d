"""Build libtb.so (the gfx950 HIP library) in-tree with hipcc."""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtb.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


NOISE = "packed-fp32-ops' is not a recognized feature"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    if r.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed: %s" % " ".join(cmd[-3:]))
    if err.strip() and verbose:
        sys.stderr.write(err + "\n")


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for a CPU-only
# check of the library's argument validation; device code is built as usual.
HOST_SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def build(verbose=False, jobs=None, lib=None, objdir=None, extra_flags=()):
    """Compile every csrc/*.hip to an object (in parallel), then link libtb.so
    (or `lib`, with objects under `objdir` and `extra_flags` on every line)."""
    from concurrent.futures import ThreadPoolExecutor
    lib = lib or LIB
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = objdir or os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra_flags)
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2) - 1), 8)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([hipcc()] + flags + ["-c", so[0], "-o", so[1]], verbose),
                    zip(srcs, objs)))
    tmp = lib + ".tmp"
    _run([hipcc()] + HIPCC_FLAGS + list(extra_flags) + ["-o", tmp] + objs, verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
