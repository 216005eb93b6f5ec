"""ctypes binding of libspecprobe (include/spec_probe.h): the measurement
kernels the benchmark uses for the HBM read ceiling and the launch floor.
Argument marshalling only; the reads run in the library's HIP kernels."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_PATH = os.path.join(_PKG, "libspecprobe.so")
EXPORTED = ["spec_probe_read", "spec_probe_read_lds", "spec_probe_empty"]

_lib = None


def load(path: str = PROBE_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m sparse_kv_attention_sink_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.spec_probe_read.argtypes = [P, SZ, I32, I32, P, P]
    lib.spec_probe_read.restype = I32
    lib.spec_probe_read_lds.argtypes = [P, SZ, I32, I32, P, P]
    lib.spec_probe_read_lds.restype = I32
    lib.spec_probe_empty.argtypes = [I32, P, P]
    lib.spec_probe_empty.restype = I32
    _lib = lib
    return lib


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ok(st: int, what: str) -> None:
    if st != 0:
        raise RuntimeError(f"{what} returned {st}")


def read(src: torch.Tensor, workgroups: int, in_flight: int, sink: torch.Tensor) -> None:
    """One read of every byte of ``src`` (register path); ``sink`` holds
    ``workgroups`` int32 words."""
    assert src.is_cuda and sink.is_cuda and sink.numel() >= workgroups
    nbytes = src.numel() * src.element_size()
    _ok(load().spec_probe_read(ctypes.c_void_p(src.data_ptr()), nbytes, workgroups, in_flight,
                               ctypes.c_void_p(sink.data_ptr()), _stream(src)), "spec_probe_read")


def read_lds(src: torch.Tensor, workgroups: int, stages: int, sink: torch.Tensor) -> None:
    """One read of every byte of ``src`` through the HBM-to-LDS copy."""
    assert src.is_cuda and sink.is_cuda and sink.numel() >= workgroups
    nbytes = src.numel() * src.element_size()
    _ok(load().spec_probe_read_lds(ctypes.c_void_p(src.data_ptr()), nbytes, workgroups, stages,
                                   ctypes.c_void_p(sink.data_ptr()), _stream(src)),
        "spec_probe_read_lds")


def empty(workgroups: int, sink: torch.Tensor) -> None:
    assert sink.is_cuda and sink.numel() >= workgroups
    _ok(load().spec_probe_empty(workgroups, ctypes.c_void_p(sink.data_ptr()), _stream(sink)),
        "spec_probe_empty")
