"""Builds the HIP library libigemmconv.so in-tree for gfx950.

The library is several translation units (the C entry points and one per
kernel family; the wide-layer family once per element type), compiled in
parallel to objects under _build/ and linked into one shared library.
"""
import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libigemmconv.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

# (object name, source, extra defines)
UNITS = [("igemm_conv", "igemm_conv.hip", [])]
for _dt in ("BF16", "FP16", "FP8"):
    _d = f"-DIGC_DT=igc::DT_{_dt}"
    UNITS += [(f"launch_band_{_dt.lower()}", "launch_band.hip", [_d]),
              (f"launch_tapfold_{_dt.lower()}", "launch_tapfold.hip", [_d]),
              (f"launch_wide_{_dt.lower()}", "launch_wide.hip", [_d]),
              (f"launch_resident_{_dt.lower()}", "launch_small.hip", [_d, "-DIGC_FAMILY=0"]),
              (f"launch_tiled_{_dt.lower()}", "launch_small.hip", [_d, "-DIGC_FAMILY=1"])]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 (v_pk_*_f32) code generation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _newest_source():
    paths = [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    paths += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    return max(os.path.getmtime(p) for p in paths)


def build(verbose: bool = False, jobs: int = None, incremental: bool = False) -> str:
    """Compile every unit and link.  incremental=True skips units whose object
    is newer than every source and header (a developer shortcut; the default
    always compiles everything)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    hipcc = _hipcc()
    newest = _newest_source() if incremental else None
    cmds = []
    objs = []
    for name, src, defs in UNITS:
        obj = os.path.join(OBJ_DIR, name + ".o")
        objs.append(obj)
        if incremental and os.path.exists(obj) and os.path.getmtime(obj) > newest:
            continue
        cmds.append([hipcc, *HIPCC_FLAGS, *defs, "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    if jobs is None:
        jobs = max(1, min(len(cmds), os.cpu_count() or 1))

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(run, c) for c in cmds]:
            f.result()
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    run(link)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    import sys
    print(build(verbose=True, incremental="--incremental" in sys.argv))
