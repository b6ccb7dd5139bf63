"""HBM read ceilings on this GPU, for comparison with the decode kernels.

    python -m paged_kv_cache_72_amd.probe.run_probes

Measurement only: loads libpa_probe.so (built by ``__graft_entry__.build()``)
and prints one markdown table of wave-contiguous reads: each wave streams its
own contiguous chunk, 16 B per lane per load, ``unroll`` loads in flight (the
best plain-read rate, the ceiling the decode kernels are compared with).

Times are medians of 30 launches bracketed by HIP events, rotating over three
buffers so that no launch finds its data in the 256 MB Infinity Cache.
"""
from __future__ import annotations

import ctypes as C
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(os.path.dirname(HERE), "libpa_probe.so")


def _lib():
    if not os.path.exists(LIB):
        raise ImportError(f"{LIB} is missing: run __graft_entry__.build()")
    L = C.CDLL(LIB)
    L.pa_probe_wave_chunk.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int32, C.c_void_p,
                                      C.c_void_p]
    return L


def _median_us(fn, n: int = 30) -> float:
    for i in range(5):
        if fn(i) != 0:
            raise RuntimeError("probe launch failed")
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]) * 1e3)


def main() -> int:
    assert torch.cuda.is_available(), "the probes need a GPU"
    L = _lib()
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    rows = []

    buf_bytes = 1 << 31
    bufs = [torch.ones(buf_bytes, dtype=torch.uint8, device="cuda") for _ in range(3)]
    sink = torch.empty(16384 * 64, dtype=torch.int32, device="cuda")
    for mib in (600, 2040):
        for waves, unroll in ((2048, 16), (3072, 4)):
            steps = (mib * 1024 // waves) // unroll * unroll
            nbytes = waves * steps * 1024
            assert nbytes <= buf_bytes and waves * 64 <= sink.numel()
            t = _median_us(lambda i: L.pa_probe_wave_chunk(bufs[i % 3].data_ptr(), waves, steps,
                                                           unroll, sink.data_ptr(), st))
            rows.append((f"wave-contiguous read, {waves} waves, {unroll} KiB in flight per wave",
                         nbytes, t))
    del bufs

    print("| probe | bytes | median µs | GB/s | % of 8 TB/s |")
    print("|---|---|---|---|---|")
    for name, b, t in rows:
        print(f"| {name} | {b} | {t:.1f} | {b / t / 1e3:.0f} | {100 * b / t / 1e3 / 8000:.1f} |")
    sys.stdout.flush()
    return 0


if __name__ == "__main__":
    sys.exit(main())
