"""ctypes binding of libddtree_rates.so (include/ddtree_rates.h): achievable-rate probes, a back-to-back bf16
MFMA loop and a read-only HBM stream, that give the box's own ceilings next to the vendor peaks.  Argument
marshalling only; not part of the verify path."""
from __future__ import annotations

import ctypes
import os

import torch

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libddtree_rates.so")
_lib = None

SIGNATURES = {
    "ddtree_rates_mfma_loop": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "ddtree_rates_mfma_loop_flops": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32]),
    "ddtree_rates_stream_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                                ctypes.c_void_p]),
}


def library_path() -> str:
    return _PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is not built; run `python -m mla_tree_verify_absorb_amd.build`")
        h = ctypes.CDLL(_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype, fn.argtypes = res, args
        _lib = h
    return _lib


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def mfma_loop(workgroups: int, iters: int, sink: torch.Tensor) -> int:
    """Enqueue the MFMA loop; returns its flop count."""
    assert sink.dtype == torch.float32 and sink.numel() >= workgroups * 4
    st = lib().ddtree_rates_mfma_loop(workgroups, iters, ctypes.c_void_p(sink.data_ptr()), _stream(sink.device))
    if st != 0:
        raise RuntimeError(f"ddtree_rates_mfma_loop failed ({st})")
    return int(lib().ddtree_rates_mfma_loop_flops(workgroups, iters))


def stream_read(src: torch.Tensor, workgroups: int, sink: torch.Tensor) -> int:
    """Enqueue one read of src; returns the bytes read."""
    nbytes = src.numel() * src.element_size()
    assert src.is_contiguous() and sink.dtype == torch.int32 and sink.numel() >= workgroups * 256
    st = lib().ddtree_rates_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, workgroups,
                                        ctypes.c_void_p(sink.data_ptr()), _stream(src.device))
    if st != 0:
        raise RuntimeError(f"ddtree_rates_stream_read failed ({st})")
    return nbytes
