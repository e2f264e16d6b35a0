"""Seeded synthetic inputs and the workload shapes of the QLoRA NF4 layer.

This module only draws random numbers and describes shapes; it holds none of
the method's arithmetic.  Both the GPU path and the CPU oracle take their
inputs from here.

Distributions (reading R9: N(0, sigma) names the standard deviation):
  W  ~ N(0, 0.02) fp32        (the frozen weight, quantized to NF4)
  X  ~ N(0, 1)    bf16        (layer input, tokens x in_features)
  A  ~ U(-1/sqrt(K), 1/sqrt(K)) bf16   (LoRA down-projection, K x r)
  B  ~ N(0, 0.01) bf16        (LoRA up-projection, r x N)
  dY ~ N(0, 1)    bf16        (upstream gradient)
Seeds: W 1000+i, X 2000+i, A 3000+i, B 4000+i, dY 5000+i for linear i.
CPU draws use numpy's PCG64; bf16 rounding of the draws uses torch's
round-to-nearest-even conversion.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Linear:
    name: str
    N: int   # out_features
    K: int   # in_features


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens
    r: int
    alpha: float
    linears: tuple = field(default_factory=tuple)
    backward: bool = True
    layers: int = 1        # repeat count of the linear set (65B: 80 layers)


def _llama(hidden: int, mlp: int):
    return (Linear("q_proj", hidden, hidden), Linear("k_proj", hidden, hidden),
            Linear("v_proj", hidden, hidden), Linear("o_proj", hidden, hidden),
            Linear("gate_proj", mlp, hidden), Linear("up_proj", mlp, hidden),
            Linear("down_proj", hidden, mlp))


WORKLOADS = {
    "tiny": Workload("tiny-512x512-T32-r8", 32, 8, 16.0, (Linear("w", 512, 512),)),
    "gemv7b": Workload("llama7b-q_proj-gemv-T4-r64", 4, 64, 16.0,
                       (Linear("q_proj", 4096, 4096),), backward=False),
    "mlp7b": Workload("llama7b-mlp-T2048-r64", 2048, 64, 16.0,
                      (Linear("gate_proj", 11008, 4096), Linear("up_proj", 11008, 4096),
                       Linear("down_proj", 4096, 11008))),
    "layer33b": Workload("llama33b-layer-T4096-r64", 4096, 64, 16.0, _llama(6656, 17920)),
    "full65b": Workload("llama65b-80layers-T512-r64", 512, 64, 16.0, _llama(8192, 22016), layers=80),
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """The fp32 values that bf16 words encode: each word is the upper half of
    the fp32 word, so the widening is exact."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weight(N: int, K: int, i: int = 0) -> np.ndarray:
    return _rng(1000 + i).normal(0.0, 0.02, size=(N, K)).astype(np.float32)


def x_bits(T: int, K: int, i: int = 0) -> np.ndarray:
    return to_bf16_bits(_rng(2000 + i).normal(0.0, 1.0, size=(T, K)))


def a_bits(K: int, r: int, i: int = 0) -> np.ndarray:
    a = 1.0 / np.sqrt(K)
    return to_bf16_bits(_rng(3000 + i).uniform(-a, a, size=(K, r)))


def b_bits(r: int, N: int, i: int = 0) -> np.ndarray:
    return to_bf16_bits(_rng(4000 + i).normal(0.0, 0.01, size=(r, N)))


def dy_bits(T: int, N: int, i: int = 0) -> np.ndarray:
    return to_bf16_bits(_rng(5000 + i).normal(0.0, 1.0, size=(T, N)))


def device_weight(out, i=0):
    """Fill the fp32 device tensor `out` with the seeded N(0, 0.02) weight of
    linear i (drawn on the device, for timing at full size)."""
    import torch
    g = torch.Generator(device=out.device)
    g.manual_seed(1000 + i)
    return out.normal_(0.0, 0.02, generator=g)


def device_inputs(T, N, K, r, i=0, device="cuda", backward=True, weight=True):
    """Seeded inputs drawn directly on the device (for timing at full size)."""
    import torch
    g = torch.Generator(device=device)
    out = {}
    if weight:
        g.manual_seed(1000 + i)
        out["W"] = torch.randn(N, K, generator=g, device=device, dtype=torch.float32) * 0.02
    g.manual_seed(2000 + i)
    out["X"] = torch.randn(T, K, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    g.manual_seed(3000 + i)
    a = 1.0 / float(np.sqrt(K))
    out["A"] = ((torch.rand(K, r, generator=g, device=device, dtype=torch.float32) * 2 - 1) * a).to(torch.bfloat16)
    g.manual_seed(4000 + i)
    out["B"] = (torch.randn(r, N, generator=g, device=device, dtype=torch.float32) * 0.01).to(torch.bfloat16)
    if backward:
        g.manual_seed(5000 + i)
        out["dY"] = torch.randn(T, N, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out
