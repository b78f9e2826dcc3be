"""Builds the HIP library libigemmconv.so in-tree for gfx950.

The library is several translation units (the C entry points and one per
kernel family and element type), compiled in parallel to objects under
_build/ and linked into one shared library.  The same sources are also built
as libigemmconv_ldspoison.so with IGC_LDS_POISON defined: a debug build whose
kernels first fill their LDS with NaN bytes, so that a read running ahead of
its data (a missing wait or barrier) shows up as NaN outputs in the tests.
"""
import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libigemmconv.so")
POISON_LIB = os.path.join(PKG, "libigemmconv_ldspoison.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

# (object name, source, extra defines)
UNITS = [("igemm_conv", "igemm_conv.hip", [])]
for _dt in ("BF16", "FP16", "FP8"):
    _d = f"-DIGC_DT=igc::DT_{_dt}"
    UNITS += [(f"launch_band_{_dt.lower()}", "launch_band.hip", [_d]),
              (f"launch_tapfold_{_dt.lower()}", "launch_tapfold.hip", [_d]),
              (f"launch_wide_{_dt.lower()}", "launch_wide.hip", [_d]),
              (f"launch_patch_{_dt.lower()}", "launch_patch.hip", [_d]),
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


def build(verbose: bool = False, jobs: int = None, incremental: bool = False,
          poison: bool = True) -> str:
    """Compile every unit and link, for the library and (poison=True) its
    LDS-poison debug build.  incremental=True skips units whose object is
    newer than every source and header (a developer shortcut; the default
    always compiles everything)."""
    hipcc = _hipcc()
    newest = _newest_source() if incremental else None
    variants = [(LIB, OBJ_DIR, [])]
    if poison:
        variants.append((POISON_LIB, os.path.join(OBJ_DIR, "ldspoison"), ["-DIGC_LDS_POISON"]))
    cmds = []
    links = []
    for lib, obj_dir, extra in variants:
        os.makedirs(obj_dir, exist_ok=True)
        objs = []
        for name, src, defs in UNITS:
            obj = os.path.join(obj_dir, name + ".o")
            objs.append(obj)
            if incremental and os.path.exists(obj) and os.path.getmtime(obj) > newest:
                continue
            cmds.append([hipcc, *HIPCC_FLAGS, *extra, *defs, "-I", INCLUDE, "-I", CSRC, "-c",
                         os.path.join(CSRC, src), "-o", obj])
        links.append((lib, [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o",
                            lib + ".tmp"]))
    if jobs is None:
        jobs = max(1, min(len(cmds), os.cpu_count() or 1))

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    with concurrent.futures.ThreadPoolExecutor(max_workers=max(jobs, 1)) as ex:
        for f in [ex.submit(run, c) for c in cmds]:
            f.result()
    for lib, link in links:
        run(link)
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    import sys
    print(build(verbose=True, incremental="--incremental" in sys.argv,
                poison="--no-poison" not in sys.argv))
