"""Measurement aid: a plain streaming read (libcsa_calib.so) that calibrates
what a read-only kernel reaches from HBM on this GPU.  Not part of the
indexer; only the benchmark uses it."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
CALIB_PATH = os.path.join(HERE, "libcsa_calib.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(CALIB_PATH):
            raise ImportError(f"{CALIB_PATH} is missing: build it with `python -m lightning_indexer_top_02_amd.build`")
        lib = ctypes.CDLL(CALIB_PATH)
        lib.csa_calib_read_stream.restype = ctypes.c_int
        lib.csa_calib_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        lib.csa_calib_read_grid.restype = ctypes.c_int
        lib.csa_calib_read_grid.argtypes = []
        _lib = lib
    return _lib


def read_stream(buf, sink):
    """Read every byte of the contiguous GPU tensor `buf` once (on torch's
    current stream); `sink` is an int32 GPU tensor of at least
    csa_calib_read_grid() entries."""
    import torch
    lib = load()
    nbytes = buf.numel() * buf.element_size()
    if not (buf.is_cuda and buf.is_contiguous() and sink.is_cuda and sink.numel() >= lib.csa_calib_read_grid()):
        raise ValueError("buf must be a contiguous GPU tensor and sink large enough")
    rc = lib.csa_calib_read_stream(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"csa_calib_read_stream failed with HIP error {rc}")
