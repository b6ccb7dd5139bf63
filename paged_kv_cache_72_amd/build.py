"""Build libpa.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m paged_kv_cache_72_amd.build [-v]

Every HIP source is compiled for gfx950 only, one object per source in
parallel, then linked into one shared library.  Packed-fp32 instruction
selection is disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import zlib

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpa.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
NOISE = "packed-fp32-ops"   # the host pass does not know the device feature


def sources():
    """Every HIP source plus the host-only C++ of the library (the block pool)."""
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) +
                  glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, what: str, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed: {what}")
    if verbose:
        for line in (res.stdout + res.stderr).splitlines():
            if line.strip() and NOISE not in line and "warning" in line and "loop not" not in line:
                print(line)


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    """Compile every source to an object (in parallel) and link ``out``."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    tag = "x%08x" % zlib.crc32(" ".join(extra).encode()) if extra else "rel"
    jobs = []
    for src in sources():
        base = os.path.basename(src)
        # the decode kernels compile as one object per (head_dim, KV format) slice
        slices = ([(f"{base}.d{d}k{kv}", [f"-DPA_DECODE_SLICE_D={d}", f"-DPA_DECODE_SLICE_KV={kv}"])
                   for d in (64, 128, 256) for kv in (0, 1, 2, 3, 4)]
                  if base == "pa_decode.hip" else [(base, [])])
        for name, defs in slices:
            obj = os.path.join(OBJ_DIR, f"{name}.{tag}.o")
            jobs.append((name, obj, [_hipcc(), *HIPCC_FLAGS, *extra, *defs, *inc, "-c", src,
                                     "-o", obj]))
    # longest first: the decode slices, then prefill
    jobs.sort(key=lambda j: (not j[0].startswith("pa_decode"), not j[0].startswith("pa_prefill")))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda j: _run(j[2], j[0], verbose), jobs))
    tmp = out + ".tmp"
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[j[1] for j in jobs],
          "-o", tmp], "link libpa.so", verbose)
    os.replace(tmp, out)
    return out


PROBE_LIB = os.path.join(HERE, "libpa_probe.so")


def build_probe(verbose: bool = False) -> str:
    """The HBM read-ceiling probe used by bench.py (measurement only)."""
    src = os.path.join(HERE, "probe", "stream_read.hip")
    _run([_hipcc(), *HIPCC_FLAGS, "-shared", src, "-o", PROBE_LIB + ".tmp"], "probe", verbose)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
