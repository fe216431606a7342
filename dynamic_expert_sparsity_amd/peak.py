"""Measured peaks of this GPU: HBM copy and read bandwidth, bf16 MFMA rate.

Thin ctypes binding of libbeam_peak.so (csrc/peak.hip).  The kernels run on
torch's current stream and are timed with events on that stream; each figure
is the best of several repetitions.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import lib as _layer_lib

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def peak_lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _layer_lib()  # the same HIP runtime as torch (checked there)
        path = os.path.join(_PKG, "libbeam_peak.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -m dynamic_expert_sparsity_amd.build`")
        L = ctypes.CDLL(path)
        L.beam_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
        L.beam_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_void_p]
        L.beam_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p,
                                     ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
        for f in (L.beam_peak_copy, L.beam_peak_read, L.beam_peak_mfma):
            f.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _best_ms(launch, reps: int) -> float:
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    return best


def measure(device, nbytes: int = 1 << 30, reps: int = 5, mfma_iters: int = 20000) -> dict:
    """Copy (read + write), read and MFMA peaks on `device`."""
    L = peak_lib()
    dev = torch.device(device)
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"peak kernel launch failed (HIP error {rc})")

    copy = lambda: check(L.beam_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, s))  # noqa: E731
    read = lambda: check(L.beam_peak_read(src.data_ptr(), nbytes, sink.data_ptr(), s))  # noqa: E731
    flops = ctypes.c_double()
    mfma = lambda: check(L.beam_peak_mfma(mfma_iters, sink.data_ptr(), ctypes.byref(flops), s))  # noqa: E731
    copy(), read(), mfma()  # warm-up
    torch.cuda.synchronize(dev)
    t_copy = _best_ms(copy, reps)
    t_read = _best_ms(read, reps)
    t_mfma = _best_ms(mfma, reps)
    del src, dst
    return {"copy_GBps": round(2 * nbytes / (t_copy * 1e-3) / 1e9, 1),
            "read_GBps": round(nbytes / (t_read * 1e-3) / 1e9, 1),
            "mfma_bf16_TFLOPs": round(flops.value / (t_mfma * 1e-3) / 1e12, 1),
            "bytes": nbytes, "reps": reps}
