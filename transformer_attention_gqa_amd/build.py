"""Build libgqa_attn.so in-tree with hipcc for gfx950.

    python -m transformer_attention_gqa_amd.build [--verbose]

Compiles every HIP source under csrc/ into one shared library next to this
file.  Each source is compiled to an object in _build/ (in parallel) and then
linked; everything is rebuilt on every call.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libgqa_attn.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "decode.hip", "measure.hip", "mla.hip", "prefill.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep packed-fp32 VALU instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    out = "\n".join(ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return out


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    _check_self_contained(tmp)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _check_self_contained(lib):
    """Fail the build if the library leaves any of its own symbols undefined
    (e.g. a kernel whose host-side launch stub was not emitted), which would
    otherwise only show when the library is loaded."""
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    res = subprocess.run([nm, "-D", "--undefined-only", lib], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True)
    if res.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}:\n{res.stdout}")
    missing = [ln.split()[-1] for ln in res.stdout.splitlines() if "_ZN3gqa" in ln]
    if missing:
        raise RuntimeError(f"{os.path.basename(lib)} leaves its own symbols undefined: {missing}")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose))


if __name__ == "__main__":
    sys.exit(main())
