"""Build the HIP library in-tree for gfx950: `python -m eagle_tree_verification_amd.build`.

Produces eagle_tree_verification_amd/libspecverify.so from csrc/*.hip with
hipcc.  Every call recompiles (object files go to _build/, which git ignores).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["abi.hip", "attention.hip", "accept.hip", "commit.hip", "tree.hip", "rope.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 vector ops are kept off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the online softmax rescales
    # them, which would otherwise cost an AGPR<->VGPR copy per element
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-result",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is noise
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
    return r.returncode, "\n".join(lines)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
        rc, out = _run(cmd)
        return src, obj, rc, out

    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, obj, rc, out in ex.map(compile_one, SOURCES):
            if out.strip() and (verbose or rc != 0):
                print(out, file=sys.stderr)
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src}")
            objs.append(obj)
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
