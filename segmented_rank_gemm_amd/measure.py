"""Binding of the measurement aids (include/lora_measure.h,
liblora_measure.so): a device-to-device copy and an in-place update with the
path's 16-byte vector accesses, the practical HBM ceilings the path's kernels
are measured against.  Not part of the multi-LoRA path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import _check, _flat_dev_bytes, _stream_handle

MEASURE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblora_measure.so")
_mlib = None


def measure_lib() -> ctypes.CDLL:
    """liblora_measure.so, loaded once (raises if it is not built)."""
    global _mlib
    if _mlib is None:
        if not os.path.exists(MEASURE_LIB_PATH):
            raise ImportError(f"{MEASURE_LIB_PATH} is missing: build it with "
                              "`python segmented_rank_gemm_amd/build.py` (hipcc, gfx950)")
        L = ctypes.CDLL(MEASURE_LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.lora_stream_copy.argtypes = [vp, vp, i64, vp]
        L.lora_stream_copy.restype = ctypes.c_int
        L.lora_stream_update.argtypes = [vp, i64, vp]
        L.lora_stream_update.restype = ctypes.c_int
        _mlib = L
    return _mlib


def lora_stream_copy(src: torch.Tensor, dst: torch.Tensor,
                     stream: Optional[torch.cuda.Stream] = None) -> None:
    """Copy all of src into the first bytes of dst (both contiguous device tensors)."""
    sp, nbytes = _flat_dev_bytes(src, "src")
    dp, dbytes = _flat_dev_bytes(dst, "dst")
    if dbytes < nbytes:
        raise ValueError("dst smaller than src")
    _check("lora_stream_copy",
           measure_lib().lora_stream_copy(sp, dp, int(nbytes), _stream_handle(stream)))


def lora_stream_update(buf: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> None:
    """Read, change and write back every byte of buf (a contiguous device tensor)."""
    bp, nbytes = _flat_dev_bytes(buf, "buf")
    _check("lora_stream_update",
           measure_lib().lora_stream_update(bp, int(nbytes), _stream_handle(stream)))
