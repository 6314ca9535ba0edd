"""Compile the HIP library for gfx950 in-tree.

``python -m dense_tiled_gemm_tgemm_amd.build`` writes
``dense_tiled_gemm_tgemm_amd/libtgemm.so`` (the GEMM, include/tgemm.h) and
``dense_tiled_gemm_tgemm_amd/libtgemm_probe.so`` (measurement aids,
include/tgemm_probe.h). The kernels of each (input type, output type,
epilogue) combination are instantiated by ``tgemm_inst.hip`` in an object of
their own; the objects compile in parallel and link with the host entry
points (``tgemm.hip``). All device code is built with packed-fp32
instructions disabled (``-packed-fp32-ops``).
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtgemm.so")
PROBE_LIB = os.path.join(PKG, "libtgemm_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# (input type, output type, epilogue) combinations: 0 binary16, 1 bfloat16, 2 fp32
COMBOS = [(ab, ct, epi) for ab in (0, 1, 2) for ct in (0, 1, 2) for epi in (0, 1)]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _jobs() -> int:
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        v = os.environ.get(var)
        if v and v.isdigit() and int(v) > 0:
            return min(int(v), 16)
    return max(1, min(os.cpu_count() or 1, 16))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l).strip()
    if verbose and err:
        sys.stderr.write(err + "\n")


def build(verbose: bool = False, extra=()) -> str:
    with tempfile.TemporaryDirectory(prefix="tgemm_build_") as tmpdir:
        units = [(os.path.join(CSRC, "tgemm.hip"), [], "tgemm.o")]
        for ab, ct, epi in COMBOS:
            units.append((os.path.join(CSRC, "tgemm_inst.hip"),
                          [f"-DTG_AB={ab}", f"-DTG_CT={ct}", f"-DTG_EPI={epi}"], f"inst_{ab}{ct}{epi}.o"))
        probe = (os.path.join(CSRC, "probe", "tgemm_probe.hip"), [], "tgemm_probe.o")
        cmds = [[HIPCC, *FLAGS, *extra, *defs, "-c", src, "-o", os.path.join(tmpdir, obj)]
                for src, defs, obj in units + [probe]]
        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        for lib, objs in ((LIB, [obj for _, _, obj in units]), (PROBE_LIB, [probe[2]])):
            _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                  *[os.path.join(tmpdir, obj) for obj in objs], "-o", lib + ".tmp"], verbose)
            os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
