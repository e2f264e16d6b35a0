"""Storage and memory accounting in closed form.  TEST INFRASTRUCTURE ONLY.

These connect the stored format to the figures the pages print:
  * double quantization saves about 0.37 bit per parameter, about 3 GB for a
    65B model (news write-up, innovations list; the Finnish article);
  * 16-bit full finetuning of LLaMA-65B needs more than 780 GB of GPU memory
    (news write-up, introduction; Finnish article);
  * LoRA with A = 100, B = 500 and r = 5 has 5*100 + 5*500 = 3000 parameters
    instead of 100*500 = 50000, and a rank-8 LoRA for 7B LLaMA is about 8 MB
    (LoRA tutorial, section on parameter efficiency).

Readings: the 780 GB figure is read as 16-bit weights and
gradients plus two fp32 Adam moments (2 + 2 + 8 bytes per parameter); the
8 MB figure as adapters on the q and v projections of the 32 layers of
LLaMA-7B (hidden 4096) stored in 16 bits.
"""

from __future__ import annotations

from .nf4 import storage_bytes

LLAMA = {
    # name: (layers, hidden, mlp)
    "7B": (32, 4096, 11008),
    "33B": (60, 6656, 17920),
    "65B": (80, 8192, 22016),
}


def linear_params(layers: int, hidden: int, mlp: int) -> int:
    """Parameters in the q, k, v, o and gate, up, down projections."""
    return layers * (4 * hidden * hidden + 3 * hidden * mlp)


def bits_per_param(n: int, double_quant_on: bool = True) -> float:
    return 8.0 * storage_bytes(n, double_quant_on) / n


def double_quant_saving_bits(n: int) -> float:
    return bits_per_param(n, False) - bits_per_param(n, True)


def full_finetune_bytes(params: float) -> float:
    return params * (2 + 2 + 8)


def lora_params(a: int, b: int, r: int) -> int:
    return r * a + r * b


def lora_qv_bytes(layers: int, hidden: int, r: int, bytes_per: int = 2) -> int:
    return layers * 2 * lora_params(hidden, hidden, r) * bytes_per
