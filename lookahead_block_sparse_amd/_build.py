"""Build liblsa.so (HIP for gfx950) in-tree with hipcc.

    python lookahead_block_sparse_amd/_build.py

Objects go to lookahead_block_sparse_amd/_build/, the library to
lookahead_block_sparse_amd/liblsa.so, and the read-bandwidth probe (probe/, used only by
bench.py --read-ceiling) to lookahead_block_sparse_amd/libprobe.so.  Every call recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "liblsa.so"
PROBE_DIR = PKG / "probe"
PROBE_LIB = PKG / "libprobe.so"
ARCH = "gfx950"

# Device code: no packed-fp32 instructions; -O3.  The host pass warns that it does not know the
# target feature, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", str(ROOT / "include"), "-I", str(CSRC),
          "-Wall", "-Wno-unused-function", "-Wno-unused-result"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found: the LSA library needs the ROCm toolchain to build")


def sources():
    return sorted(list(CSRC.glob("*.hip")) + list(CSRC.glob("*.cpp")))


def _compile(src: Path) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, "-c", str(src), "-o", str(obj)]
    if src.suffix == ".cpp":
        cmd = [hipcc(), *COMMON, "-x", "hip", *DEVICE_FLAGS, "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src.name} failed:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build_probe(verbose: bool = True) -> Path:
    """libprobe.so: the read-bandwidth probe (measurement only; not part of liblsa.so)."""
    BUILD.mkdir(exist_ok=True)
    src = PROBE_DIR / "read_probe.hip"
    obj = _compile(src)
    tmp = PROBE_LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libprobe.so failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}", file=sys.stderr)
    return PROBE_LIB


def build(verbose: bool = True) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max(1, min(len(srcs) + 1, os.cpu_count() or 1))) as ex:
        probe = ex.submit(build_probe, verbose)
        objs = list(ex.map(_compile, srcs))
        probe.result()
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs), "-lpthread"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking liblsa.so failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
