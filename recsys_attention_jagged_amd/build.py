"""Build libgdpa.so (gfx950) in-tree with hipcc.

    python -m recsys_attention_jagged_amd.build [--jobs N] [--verbose]

Every HIP translation unit is compiled for gfx950 only.  Packed-fp32 VALU
instructions are disabled for all device code; MFMA instructions use the VGPR
form.  Objects go to
recsys_attention_jagged_amd/_build/, the library to recsys_attention_jagged_amd/libgdpa.so.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdpa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA results in VGPRs (gfx950 has one register file): no AGPR copies
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-Wno-unused-command-line-argument"]

# marks a unit compiled without the VGPR form of MFMA results
AGPR_ACC = "<agpr-acc>"

# (output object, source, extra flags)
UNITS = [("plan.o", "plan.cpp", []),
         ("api.o", "api.cpp", []),
         ("fp32.o", "fp32.hip", []),
         ("partials.o", "partials.hip", []),
         ("jfa.o", "jfa.hip", []),
         ("norm.o", "norm.hip", []),
         ("noalloc.o", "noalloc.hip", [])]
for _d in (32, 64, 128):
    UNITS.append((f"fwd_d{_d}.o", "fwd_bf16.hip", [f"-DGDPA_D={_d}"]))
    UNITS.append((f"fused_d{_d}.o", "bwd_fused.hip", [f"-DGDPA_D={_d}"]))
    if _d < 128:
        UNITS.append((f"bwd_d{_d}.o", "bwd_bf16.hip", [f"-DGDPA_D={_d}"]))
# d = 128: the dQ and dK/dV kernels in objects of their own.  The dK/dV kernel
# (K, V, dK and dV held per wave: more than the 256 VGPRs) keeps its MFMA
# accumulators in AGPRs; with them in VGPRs the compiler parks K and V in AGPRs
# instead, copies them back every step and waits on each operand read.
UNITS.append(("bwd_dq_d128.o", "bwd_bf16.hip", ["-DGDPA_D=128", "-DGDPA_BWD_PART=1"]))
UNITS.append(("bwd_kv_d128.o", "bwd_bf16.hip", ["-DGDPA_D=128", "-DGDPA_BWD_PART=2", AGPR_ACC]))
# d = 128: the 16-row two-wave dK/dV kernel (MFMA results in VGPRs)
UNITS.append(("bwd16_d128.o", "bwd16.hip", []))


# the clock-probe library (GDPA_BIN_CLOCK): every kernel stamps the start and the end
# of each bin's walk; a separate file and build folder, never loaded by default
LIB_BIN_CLOCK = os.path.join(PKG, "libgdpa_binclock.so")


def _compile(unit, verbose, build_dir=BUILD, defines=()):
    obj, src, extra = unit
    common = list(COMMON) + list(defines)
    if AGPR_ACC in extra:
        i = common.index("-amdgpu-mfma-vgpr-form")
        del common[i - 1:i + 1]
        extra = [e for e in extra if e != AGPR_ACC]
    cmd = [HIPCC, *common, *extra, "-c", os.path.join(CSRC, src), "-o", os.path.join(build_dir, obj)]
    t0 = time.time()
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (p.stderr or "").splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compiling {src} {' '.join(extra)} failed:\n{err}")
    if verbose:
        print(f"  {obj}: {time.time() - t0:.1f}s", flush=True)
        if err.strip():
            print(err)
    return obj


def build(jobs: int = 0, verbose: bool = False, bin_clock: bool = False) -> str:
    """Compile every unit and link the library (bin_clock: the clock-probe library);
    returns its path."""
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    build_dir, lib, defines = (BUILD + "_binclock", LIB_BIN_CLOCK, ["-DGDPA_BIN_CLOCK"]) if bin_clock else \
        (BUILD, LIB, [])
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(UNITS), os.cpu_count() or 4, 16)
    t0 = time.time()
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose, build_dir, defines), UNITS))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + [os.path.join(build_dir, o) for o in objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} in {time.time() - t0:.1f}s", flush=True)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--bin-clock", action="store_true",
                    help="build the clock-probe library (libgdpa_binclock.so) instead")
    args = ap.parse_args(argv)
    build(args.jobs, args.verbose, args.bin_clock)


if __name__ == "__main__":
    main(sys.argv[1:])
