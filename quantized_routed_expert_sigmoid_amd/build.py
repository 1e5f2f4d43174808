"""Builds libcolibri.so (the gfx950 HIP library behind include/colibri.h) in-tree,
and libcolibri_debug.so, the same sources with COLI_DEBUG_PARTIALS (the
test-only build of include/colibri_debug.h, which also dumps block partials).

    python -m quantized_routed_expert_sigmoid_amd.build
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcolibri.so")
DEBUG_LIB = os.path.join(PKG, "libcolibri_debug.so")
# measurement kernels of the benchmark (include/colibri_probes.h)
PROBES_LIB = os.path.join(PKG, "libcolibri_probes.so")
PROBES_SRC = "probes.hip"

SOURCES = ["ffn_gemv.hip", "ffn_mfma.hip", "api.hip", "q8_router.hip", "dispatch.hip", "tier.hip",
           "tier_kernels.hip", "expert_cache.cpp"]

ARCH = "gfx950"
# -ffp-contract=off: every fused multiply-add in the kernels is an explicit
# fma, which the layer's canonical fold and exp depend on.  Packed fp32
# instructions are disabled for all device code.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]


# The matrix-core kernels keep MFMA results in ordinary VGPRs (no
# accumulation-register copies between the MFMA and the fp32 fold).
EXTRA = {"ffn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(job) -> str:
    src, debug = job
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ("_debug.o" if debug else ".o"))
    cmd = ["hipcc", *FLAGS, *(["-DCOLI_DEBUG_PARTIALS"] if debug else []), *EXTRA.get(src, []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Compiles both libraries (the largest sources first, so that the two
    builds of each run side by side)."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, debug) for src in SOURCES for debug in (False, True)] + [(PROBES_SRC, False)]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, jobs))
    _link([o for o, (src, d) in zip(objs, jobs) if not d and src != PROBES_SRC], LIB)
    _link([o for o, (_, d) in zip(objs, jobs) if d], DEBUG_LIB)
    _link([o for o, (src, _) in zip(objs, jobs) if src == PROBES_SRC], PROBES_LIB)
    if verbose:
        print(f"built {LIB}, {DEBUG_LIB} and {PROBES_LIB}")
    return LIB


if __name__ == "__main__":
    build()
