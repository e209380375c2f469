"""Build libkda.so in-tree with hipcc for gfx950."""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
# measurement kernels of the benchmark (achievable HBM and matrix-core rates),
# a library of their own beside libkda
PEAKS_SRC = os.path.join(CSRC, "probe", "peaks.hip")
PEAKS_LIB = os.path.join(PKG, "libkda_peaks.so")
SOURCES = ["kda_api.cpp", "kda_sizes.cpp", "chunk_fwd.hip", "chunk_fwd_bf16.hip",
           "recurrent_step.hip", "backward.hip", "bwd_chunk.hip", "gdn2_step.hip",
           "gdn2_chunk.hip", "chunk_split.hip"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = os.path.join(rocm, "bin", "hipcc")
    return exe if os.path.exists(exe) else (shutil.which("hipcc") or "hipcc")


def build(verbose=False):
    """Compile every source to an object in parallel, then link libkda.so."""
    common = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
              # keep the compiler from forming packed fp32 ALU ops
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(PKG, "..", "include")]
    with tempfile.TemporaryDirectory(prefix="kda_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc()] + common + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (src, res.stderr))
            return obj
        with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
            peaks = ex.submit(_build_peaks, common)
            objs = list(ex.map(compile_one, SOURCES))
            peaks.result()
        out = LIB + ".tmp%d" % os.getpid()
        cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n%s" % res.stderr)
        os.replace(out, LIB)
    return LIB


def _build_peaks(common):
    out = PEAKS_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + common + ["-shared", PEAKS_SRC, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (PEAKS_SRC, res.stderr))
    os.replace(out, PEAKS_LIB)


if __name__ == "__main__":
    print(build(verbose=True))
