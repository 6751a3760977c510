"""Build libgdr.so (HIP, gfx950) in-tree with hipcc: one object per source, compiled in
parallel, then linked."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgdr.so")
SOURCES = ["gdr_api.hip", "gdr_f32_split.hip", "gdr_kda_split.hip"]

# Packed fp32 ops stay off: the compiler must not form v_pk_* fp32 instructions.
# MFMA accumulators are placed in ordinary vector registers where they fit
# (-amdgpu-mfma-vgpr-form): the kernels scale, convert and store them with vector
# instructions, which otherwise copy them out of the accumulator registers first.
HIPCC_FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form",
               "-Wall", "-Wno-unused-function"]
NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    return r.returncode, err


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="gdr_build_") as tmp:
        cmds, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            cmds.append([hipcc] + HIPCC_FLAGS + inc +
                        ["-c", os.path.join(HERE, "csrc", src), "-o", obj])
        if verbose:
            for c in cmds:
                print(" ".join(c), file=sys.stderr)
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, err), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
        link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
        if verbose:
            print(" ".join(link), file=sys.stderr)
        rc, err = _run(link)
        if rc != 0:
            raise RuntimeError(f"hipcc link failed ({rc}):\n{err}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
