"""Build libtsa.so in-tree for gfx950 with hipcc (one object per source, compiled in parallel)."""

import concurrent.futures as cf
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed float32 ops stay off (hipcc's host pass warns that it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src, obj, extra):
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stderr}")
    return r.stderr


def build(extra=(), verbose=False, lib_path=LIB, obj_dir=None):
    """Compile every HIP/C++ source of the library and link libtsa.so (or lib_path, with the objects
    in obj_dir, for a separately instrumented copy).  Returns the library path."""
    out = obj_dir or os.path.join(ROOT, "_build")
    os.makedirs(out, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(out, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        logs = list(ex.map(lambda so: _compile(so[0], so[1], list(extra)), zip(srcs, objs)))
    if verbose:
        for s, log in zip(srcs, logs):
            print(f"== {os.path.basename(s)}\n{log}")
    tmp = lib_path + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    import sys
    print(build(extra=sys.argv[1:], verbose=True))
