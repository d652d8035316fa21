"""Moving generated bf16 bit patterns to and from the device (torch tensors).

No arithmetic: bits go up as int16 and are reinterpreted as bfloat16, and come
back the same way.  Used by the benchmark and the GPU tests alike.
"""

from __future__ import annotations

import numpy as np


def to_dev_bf16(bits: np.ndarray):
    """Upload raw bfloat16 bit patterns (uint16) as a device bfloat16 tensor."""
    import torch

    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).cuda().view(torch.bfloat16)


def from_dev_bf16(t) -> np.ndarray:
    """Raw bit patterns (uint16) of a device bfloat16 tensor."""
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
