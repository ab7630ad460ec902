"""ctypes binding of the measured-ceiling probes (``include/qlora_peaks.h``,
``libqlora_peaks.so``), used by the benchmark; argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_peaks.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run qlora_fine_tuning_nf4_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.qlora_peak_read.restype = i32
        L.qlora_peak_read.argtypes = [vp, sz, i32, vp, vp]
        L.qlora_peak_copy.restype = i32
        L.qlora_peak_copy.argtypes = [vp, vp, sz, vp]
        L.qlora_peak_mfma.restype = i32
        L.qlora_peak_mfma.argtypes = [i32, vp, vp]
        L.qlora_peak_mfma_flops.restype = ctypes.c_double
        L.qlora_peak_mfma_flops.argtypes = [i32]
        _lib = L
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ok(st, what):
    if st != 0:
        raise RuntimeError(f"{what} failed with status {st}")


def read(buf: torch.Tensor, contiguous: bool, sink: torch.Tensor) -> None:
    _ok(lib().qlora_peak_read(buf.data_ptr(), buf.numel() * buf.element_size(), int(contiguous),
                              sink.data_ptr(), _stream()), "qlora_peak_read")


def copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    _ok(lib().qlora_peak_copy(src.data_ptr(), dst.data_ptr(), n, _stream()), "qlora_peak_copy")


def mfma(iters: int, sink: torch.Tensor) -> None:
    _ok(lib().qlora_peak_mfma(int(iters), sink.data_ptr(), _stream()), "qlora_peak_mfma")


def mfma_flops(iters: int) -> float:
    return float(lib().qlora_peak_mfma_flops(int(iters)))
