"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method: it draws normal samples and
converts them to bf16 with torch's own float32 -> bfloat16 cast (round to
nearest even), nothing else.  Both the CPU oracle and the HIP path consume
what it produces.

Recipe (stand-ins for the trained weights and hidden states of the dense
20B-32B decoders the pages run):
* weights: float32 standard normal * float32(0.02), cast to bf16;
* activations: float32 standard normal, cast to bf16.

Host draws use numpy's PCG64 seeded with [2026, stream, tensor_id], where
`stream` numbers a family of inputs (one per workload, 0-4, and others for
test fixtures); device draws (for the 48-layer sweep, too large to draw on the
host) use torch's generator on the device, seeded with
2026 * 1_000_003 + stream * 1_000 + tensor_id.  A tensor is always drawn the
same way for a given (stream, tensor_id).
"""

import numpy as np

WEIGHT_STD = np.float32(0.02)
SEED = 2026


def _rng(stream, tensor_id):
    return np.random.default_rng([SEED, int(stream), int(tensor_id)])


def _bf16_bits_torch(f32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def host_normal_f32(stream, tensor_id, shape, scale=None):
    g = _rng(stream, tensor_id)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if scale is not None:
        a = (a * np.float32(scale)).astype(np.float32)
    return a


def weight_bits(stream, tensor_id, n_out, k):
    """bf16 bit patterns (uint16 [n_out][k]) of a seeded ~N(0, 0.02) weight matrix."""
    return _bf16_bits_torch(host_normal_f32(stream, tensor_id, (n_out, k), WEIGHT_STD))


def act_bits(stream, tensor_id, shape):
    """bf16 bit patterns of seeded ~N(0, 1) activations of the given shape."""
    return _bf16_bits_torch(host_normal_f32(stream, tensor_id, shape))


def device_seed(stream, tensor_id):
    return SEED * 1_000_003 + int(stream) * 1_000 + int(tensor_id)


def device_normal_bf16(stream, tensor_id, shape, scale=None, device="cuda"):
    """A seeded bf16 tensor drawn on the device (torch generator on that device)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(stream, tensor_id))
    a = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if scale is not None:
        a.mul_(float(np.float32(scale)))
    return a.to(torch.bfloat16)


def device_weight(stream, tensor_id, n_out, k, device="cuda"):
    return device_normal_bf16(stream, tensor_id, (n_out, k), WEIGHT_STD, device)
