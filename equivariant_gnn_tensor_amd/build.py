"""Build libetpc.so for gfx950 with hipcc (in-tree, parallel, one object per source).

    python equivariant_gnn_tensor_amd/build.py [--force] [--jobs N]
        [--define NAME=VALUE ...] [--flag HIPCC_FLAG ...] [--build-dir DIR --lib PATH]

Objects go to <repo>/_build/, the library to equivariant_gnn_tensor_amd/_lib/libetpc.so.
Without --force, a source is recompiled only when it or any header is newer than
its object.  --define passes tuning macros (e.g. ETPC_BWD_PREFETCH=3) to every
kernel source; use it with a separate --build-dir and --lib so the default
library is left alone (the binding loads $ETPC_LIBRARY when set).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libetpc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results and accumulators in ordinary VGPRs: the traversals read their
    # 4x4x1 results with VALU code, and AGPR<->VGPR copies cost more than they save
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


GENERATOR = "gen_cg.cpp"
CG_INC = os.path.join(CSRC, "cg_tables.inc")


def _sources():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    return [s for s in srcs if os.path.basename(s) != GENERATOR]


def _gen_cg_tables(force: bool) -> None:
    """Compile and run the coupling-table generator (host code) -> csrc/cg_tables.inc."""
    gen_src = [os.path.join(CSRC, GENERATOR), os.path.join(CSRC, "plan.cpp")]
    exe = os.path.join(BUILD, "gen_cg")
    newest_src = max(os.path.getmtime(p) for p in gen_src + [os.path.join(CSRC, "plan.hpp")])
    if not force and os.path.exists(CG_INC) and os.path.getmtime(CG_INC) >= newest_src:
        return
    cmd = [HIPCC, "-xhip", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), *gen_src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the coupling-table generator failed:\n" + r.stderr)
    r = subprocess.run([exe, CG_INC + ".tmp"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("coupling-table generator failed:\n" + r.stderr)
    os.replace(CG_INC + ".tmp", CG_INC)


def _headers():
    return (glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(CSRC, "*.inc"))
            + glob.glob(os.path.join(ROOT, "include", "*.h")))


def _compile(src: str, force: bool, newest_header: float, build_dir: str, defines, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    if not force and os.path.exists(obj):
        t = os.path.getmtime(obj)
        if t >= os.path.getmtime(src) and t >= newest_header:
            return obj
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(force: bool = False, jobs: int = 0, verbose: bool = True, defines=(), build_dir: str = BUILD,
          lib: str = LIB, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(os.path.dirname(os.path.abspath(lib)), exist_ok=True)
    _gen_cg_tables(force)
    srcs = _sources()
    hdr = max((os.path.getmtime(h) for h in _headers()), default=0.0)
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, force, hdr, build_dir, defines, extra), srcs))
    newest = max(os.path.getmtime(o) for o in objs)
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < newest:
        tmp = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stderr)
        os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--define", action="append", default=[])
    ap.add_argument("--build-dir", default=BUILD)
    ap.add_argument("--lib", default=LIB)
    ap.add_argument("--flag", action="append", default=[], help="extra hipcc flag for every kernel source")
    a = ap.parse_args()
    if (a.define or a.flag or a.lib != LIB) and (a.build_dir == BUILD or a.lib == LIB):
        ap.error("--define, --flag and --lib need their own --build-dir and --lib")
    build(force=a.force, jobs=a.jobs, defines=a.define, build_dir=a.build_dir, lib=a.lib, extra=a.flag)


if __name__ == "__main__":
    main()
