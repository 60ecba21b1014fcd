"""Build librope_fa.so (HIP, gfx950 only) in-tree with hipcc.

``python -m rope_flashattention_amd.build`` or ``build()`` from Python.  The library
lands next to this file, where the binding loads it.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librope_fa.so")
SOURCES = ["api.cpp", "rope_tables.hip", "rope_qk.hip", "flash_fwd.hip", "flash_fwd_bf16.hip", "flash_fwd_f16.hip",
           "kv_cache.hip", "decode.hip", "flash_bwd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed-fp32 VALU instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
_NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source to an object (in parallel), then link the shared library."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="rope_fa_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(src)[0] + ".o") for src in SOURCES]
        cmds = [[hipcc(), *HIPCC_FLAGS, *(extra_flags or []), *inc, "-c", os.path.join(CSRC, src), "-o", obj]
                for src, obj in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-shared", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
