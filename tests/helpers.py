"""Shared helpers for the tests: host<->device conversions and comparisons.
Holds none of the method's arithmetic."""
import numpy as np
import torch

import synth


def dev_bf16(bits: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def mask_to_dev(mask_u64: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(mask_u64).view(np.int64)).to(device)


def mask_to_host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


def bf16_f32(bits) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits)
