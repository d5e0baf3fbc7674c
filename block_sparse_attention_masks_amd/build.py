"""Build libvsa.so (the HIP kernels and their C ABI) for gfx950, in-tree.

Usage: python -m block_sparse_attention_masks_amd.build  [-v] [--sanitize]
Every .hip file under csrc/ is compiled by hipcc to an object, in parallel, and
the objects are linked into block_sparse_attention_masks_amd/libvsa.so.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libvsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unknown-pragmas",
    # keep the compiler from emitting packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    msgs = [ln for ln in r.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln
            and "is not a recognized feature for this target" not in ln]
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the argument-validation layer
# (the device code is built as usual): each flag applies to the host compilation only.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
SANITIZED_LIB = os.path.join(PKG, "_build", "sanitize", "libvsa.so")


def build(verbose=False, sanitize=False):
    """Compile every csrc/*.hip for gfx950 and link libvsa.so in the package directory.  With
    sanitize=True the host code is instrumented and the library goes to _build/sanitize/ instead:
    point VSA_LIB at it and preload the ASan runtime into the (uninstrumented) interpreter, with
    ASAN_OPTIONS=detect_leaks=0 since CPython's own allocations are not freed at exit."""
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    out_dir = os.path.join(PKG, "_build", "sanitize") if sanitize else os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    flags = FLAGS + (SANITIZE if sanitize else [])
    objs = [os.path.join(out_dir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _run([HIPCC, *flags, "-c", so[0], "-o", so[1]], verbose),
                    zip(srcs, objs)))
    lib = SANITIZED_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    link = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"] \
        if sanitize else []
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link, "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
