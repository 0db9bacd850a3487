"""Helpers for GPU tests: numpy inputs -> device tensors, case banners."""

from __future__ import annotations

import sys

import numpy as np


def banner(msg: str) -> None:
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def dev_f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def bf16_bits_from_f64(x) -> np.ndarray:
    """float64 -> bf16 bits via float32 (round to nearest even); -inf stays -inf."""
    from speculative_sampling_verification_row_amd.inputs import bf16_bits
    return bf16_bits(np.asarray(x, dtype=np.float32))
