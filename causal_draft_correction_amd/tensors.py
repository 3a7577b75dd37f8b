"""Host-array to device-tensor marshalling (bf16 bit patterns become torch.bfloat16)."""
from __future__ import annotations

import numpy as np
import torch


def device_tensor(a, device="cuda"):
    """numpy array -> contiguous device tensor; uint16 arrays are bfloat16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def head_weights_to_device(weights, device="cuda") -> dict:
    """An object with W1, W2, W_ih, W_hh, b_ih, b_hh, E numpy arrays -> dict of device tensors."""
    out = {}
    for k in ("W1", "W2", "W_ih", "W_hh", "b_ih", "b_hh", "E"):
        a = getattr(weights, k)
        out[k] = None if a is None else device_tensor(a, device)
    return out
