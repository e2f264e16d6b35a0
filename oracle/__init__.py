"""CPU oracle for the QLoRA NF4 linear layer -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously correct fp64/fp32 implementation of
what the QLoRA hot path computes: the 4-bit NormalFloat (NF4) codebook,
blockwise absmax quantization, double quantization of the absmax constants,
dequantization to the bf16 compute dtype, and the forward and backward pass of
a frozen NF4 linear layer with a LoRA adapter.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The
product library (``bit_nf4_quantized_21_amd``) never imports it and shares no
code, table or constant generator with it: the GPU library builds its own
codebook on the host from its own inverse-normal routine, and the tests check
that the two tables agree bit for bit.

Sources (the web pages about QLoRA this build works from):
  * "QLoRA: Efficient Finetuning of Quantized LLMs" (paper page on fugumt.com),
    Abstract -- frozen 4-bit base, gradients only into LoRA; (a) NF4, (b)
    double quantization.
  * The Chinese news write-up of QLoRA (chatgpt.dh666.cn), section listing the
    innovations -- NF4 is information-theoretically optimal for normally
    distributed data and beats 4-bit ints and floats; double quantization
    saves about 0.37 bit per parameter (about 3 GB at 65B).
  * The QLoRA project page (aibars.net), configuration example -- 4-bit load,
    NF4, double quantization on, bf16 compute dtype.
  * The LoRA tutorial (szsimon.cn), sections on the weight update and on
    parameter efficiency -- h = Wx + dW x with dW = W_A W_B, W frozen.

Where the pages are silent (codebook construction, block sizes, 8-bit
constant format, nibble order, tie rules) each module states the reading it
takes.

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""

from .nf4 import (  # noqa: F401
    BLOCK, BLOCK2, codebook, midpoints, quantize_nf4, pack_codes, unpack_codes,
    double_quant, dequant_scales, dequantize, bf16_round, bf16_bits_to_f32,
    f32_to_bf16_bits,
)
from .lora import linear_fwd, linear_bwd  # noqa: F401
from .compare import check_close, rel_fro, max_excess  # noqa: F401
