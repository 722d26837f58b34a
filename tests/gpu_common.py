"""Helpers shared by the GPU parity tests: device upload and oracle conversions."""

import numpy as np

import oracle

DEV = "cuda"


def to_dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev_u8(buf):
    import torch
    return torch.from_numpy(np.ascontiguousarray(buf, dtype=np.uint8)).to(DEV)


def bits_of(t):
    """uint16 bit patterns of a bf16 device tensor, on the host."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits):
    return oracle.f32_from_bf16_bits(bits).astype(np.float64)


def say(msg):
    print(msg, flush=True)
