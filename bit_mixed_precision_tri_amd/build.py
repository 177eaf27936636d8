"""Build libtri.so (the gfx950 HIP library) in-tree with hipcc."""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libtri.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Per-source extra flags.  The prefill GEMM carries sixteen 16-register MFMA accumulators
# around its K loop; LLVM's default splitting of wide loop-carried vectors into 32-bit pieces
# makes the register allocator shuttle them between accumulation and vector registers.
EXTRA_FLAGS = {
    "tri_gemm.hip": ["-mllvm", "-amdgpu-codegenprepare-break-large-phis=0"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose=False):
    """Compile every HIP source into _lib/libtri.so (always recompiles)."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(LIB_DIR, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tag = "%d" % os.getpid()
    objs = []
    cmds = []
    for src in sources():
        obj = os.path.join(LIB_DIR, os.path.basename(src) + "." + tag + ".o")
        objs.append(obj)
        cmds.append([hipcc] + HIPCC_FLAGS + EXTRA_FLAGS.get(os.path.basename(src), []) +
                    ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj])
    try:
        with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp" + tag
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
