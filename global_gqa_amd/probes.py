"""Roofline probes: the dense bf16 MFMA rate, the shader clock under that
load, and the HBM read rate, measured on the card in use (libg3probe.so).
They calibrate the kernels' fraction of peak; the published peaks stay the
targets."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_PKG, "libg3probe.so")
_lib = None


def _probe_lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with `python -m global_gqa_amd.build`")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        d = ctypes.POINTER(ctypes.c_double)
        L.g3probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, d, d, d]
        L.g3probe_mfma.restype = ctypes.c_int
        L.g3probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int, d,
                                     d]
        L.g3probe_stream.restype = ctypes.c_int
        _lib = L
    return _lib


def mfma_ceiling(workgroups: int = 512, iters: int = 4000, reps: int = 5) -> dict:
    """Best-of-reps dense bf16 MFMA rate (TFLOP/s) of 32x32x16 chains in
    every wave, and the median shader clock (GHz) over that launch."""
    t, c, ms = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    rc = _probe_lib().g3probe_mfma(workgroups, iters, reps, ctypes.byref(t), ctypes.byref(c), ctypes.byref(ms))
    if rc != 0:
        raise RuntimeError(f"g3probe_mfma failed: {rc}")
    return {"tflops": t.value, "clock_ghz": c.value, "ms": ms.value, "workgroups": workgroups,
            "mfma_per_wave": iters * 32}


def hbm_read_ceiling(nbytes: int = 2 << 30, reps: int = 5) -> dict:
    """Best HBM read rate (GB/s) over a device buffer of nbytes (well past
    the 256 MB Infinity Cache), over a few access patterns: grid-stride, and
    each workgroup streaming its own contiguous share (as a decode split
    does), at several grid sizes."""
    import torch

    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    runs = []
    try:
        for blocks, wgs in ((0, 4096), (1, 1024), (1, 2048), (1, 4096)):
            g, ms = ctypes.c_double(), ctypes.c_double()
            rc = _probe_lib().g3probe_stream(ctypes.c_void_p(buf.data_ptr()), nbytes, wgs, reps, blocks,
                                             ctypes.byref(g), ctypes.byref(ms))
            if rc != 0:
                raise RuntimeError(f"g3probe_stream failed: {rc}")
            runs.append({"pattern": "per-workgroup blocks" if blocks else "grid-stride", "workgroups": wgs,
                         "gbps": g.value, "ms": ms.value})
        torch.cuda.synchronize()
    finally:
        del buf
    best = max(runs, key=lambda r: r["gbps"])
    return {"gbps": best["gbps"], "bytes": nbytes, "best": best, "runs": runs}
