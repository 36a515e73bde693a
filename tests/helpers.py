"""Shared helpers for the GPU tests: moving seeded bf16 bit patterns to the device and
back.  No step of the method lives here."""
import numpy as np
import torch

DEV = "cuda:0"


def to_dev(bits):
    """uint16 bf16 bit patterns (numpy) -> torch bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_host_u8(t):
    return t.cpu().numpy()


def bf16_bits_of(t):
    """torch bfloat16 tensor -> uint16 numpy bit patterns."""
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def f32_to_bf16_rne_bits(x):
    """float32 numpy array -> bf16 bits, round to nearest even (via PyTorch's cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
