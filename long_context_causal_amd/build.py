"""Builds ``libcpattn.so`` (HIP kernels + C ABI) for gfx950 with hipcc.

Every ``csrc/*.hip`` and ``csrc/*.cpp`` is compiled to an object under
``_build/`` at the repository root, then linked in-tree into
``long_context_causal_amd/libcpattn.so``.  ``build()`` always recompiles;
``ensure_built()`` compiles only when no library exists.
"""
import concurrent.futures
import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcpattn.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcpattn.so)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
    # keep packed-fp32 instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-kernel resource remarks: the build refuses any kernel that spills to
# scratch.  The attention kernels complete their direct global -> LDS copies
# with hand-counted vmcnt waits, which are only right while the compiler
# issues no vector-memory instruction of its own inside their loops; a spill
# would add such instructions silently.
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def scratch_users(remarks: str) -> list:
    """(kernel, bytes per lane) of every kernel whose remarks report a
    nonzero ScratchSize."""
    found, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None and int(m.group(1)) > 0:
            found.append((name, int(m.group(1))))
    return found


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    device = src.endswith(".hip")
    cmd = [hipcc(), *COMMON, *([RESOURCE_REMARKS] if device else []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "remark:")
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    spills = scratch_users(res.stderr)
    if spills:
        raise RuntimeError(f"{src}: kernels use scratch memory (register spills): {spills}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) +
                  glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
