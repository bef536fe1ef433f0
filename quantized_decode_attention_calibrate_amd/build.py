"""Build libkvq.so (all HIP sources in csrc/) for gfx950 with hipcc, in-tree,
libkvq_check.so, the same sources with -DKVQ_CHECK=1 (device-side checks
of the caller's block ids, slots and sequence lengths; kvq_check_flags), and
libkvq_trace.so, with -DKVQ_TRACE=1 (phase timestamps; kvq_trace_set).

    python -m quantized_decode_attention_calibrate_amd.build

Flags: -O3, no fast-math (the quantize step is an IEEE fp32 division),
packed-fp32 VALU ops disabled, MFMA accumulators in VGPRs, code object v5
(loads under the HIP runtime that PyTorch ships).  The libraries bind their own symbols first
(-Bsymbolic), so they can be loaded into one process.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq.so")
LIB_CHECK = os.path.join(PKG, "libkvq_check.so")
LIB_TRACE = os.path.join(PKG, "libkvq_trace.so")
BUILD_DIR = os.path.join(ROOT, "_build")
# variant -> (library, extra compile flags, object directory)
VARIANTS = {
    "release": (LIB, [], BUILD_DIR),
    "check": (LIB_CHECK, ["-DKVQ_CHECK=1"], os.path.join(BUILD_DIR, "check")),
    "trace": (LIB_TRACE, ["-DKVQ_TRACE=1"], os.path.join(BUILD_DIR, "trace")),
}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs, not AGPRs: the softmax and the rescale read
    # every accumulator each chunk, and AGPR operands cost a v_accvgpr move
    # each way (about 14% of the single-query decode loop's instructions)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-fno-fast-math", "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra=(), obj_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Every library variant (the release one's path is returned)."""
    srcs = sources()
    jobs = []
    for lib, extra, obj_dir in VARIANTS.values():
        os.makedirs(obj_dir, exist_ok=True)
        jobs += [(src, extra, obj_dir) for src in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    for vi, (lib, _, _) in enumerate(VARIANTS.values()):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
               *objs[vi * len(srcs):(vi + 1) * len(srcs)], "-Wl,-rpath,/opt/rocm/lib", "-Wl,-Bsymbolic",
               f"-Wl,-soname,{os.path.basename(lib)}"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib}")
    return LIB


def is_stale() -> bool:
    libs = [lib for lib, _, _ in VARIANTS.values()]
    if not all(os.path.exists(lib) for lib in libs):
        return True
    t = min(os.path.getmtime(lib) for lib in libs)
    deps = sources() + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    deps.append(os.path.join(INCLUDE, "kvq.h"))
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    build()
    sys.exit(0)
