"""Shared pytest configuration: the ``gpu`` marker and host-side tensor helpers."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def bits16(t: torch.Tensor) -> np.ndarray:
    """Raw BF16 bit patterns of a tensor (any device) as a host uint16 array."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits8(t: torch.Tensor) -> np.ndarray:
    """Raw byte codes of an FP8 / uint8 tensor as a host uint8 array."""
    t = t.detach().cpu().contiguous()
    if t.dtype != torch.uint8:
        t = t.view(torch.uint8)
    return t.numpy()


def values(t: torch.Tensor) -> np.ndarray:
    """Host float64 values of a BF16 or FP32 tensor (BF16 decoded by the oracle's codec)."""
    from oracle.formats import bf16_bits_to_f64
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(bits16(t))
    return t.detach().cpu().double().numpy()
