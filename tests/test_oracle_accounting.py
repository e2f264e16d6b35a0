"""Pins of the stored format and the layer's parameter counts against the
figures the pages print (tests/golden/page_figures.json) and the workload
descriptions state (tests/golden/workload_figures.json), and of NF4's
quantization error against the Int4 and FP4 types the pages compare it with."""

import json
import os

import numpy as np
import pytest

from oracle import accounting, baselines, nf4

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
WORKLOAD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "workload_figures.json")))


def test_bits_per_param_from_actual_outputs():
    """Count the bytes the oracle actually produces for a tensor."""
    w = np.random.Generator(np.random.PCG64(0)).normal(0, 0.02, 64 * 256 * 4).astype(np.float32)
    codes, q8, s2, absmax = nf4.quantize_all(w)
    with_dq = 8 * (codes.nbytes + q8.nbytes + s2.nbytes) / w.size
    without = 8 * (codes.nbytes + absmax.nbytes) / w.size
    assert with_dq == 4 + 8 / 64 + 32 / (64 * 256) == 4.126953125
    assert without == 4.5
    assert with_dq == accounting.bits_per_param(w.size)


def test_double_quant_saving_matches_page():
    g = GOLD["double_quant_saving_bits_per_param"]
    saving = accounting.double_quant_saving_bits(1 << 24)
    assert saving == 0.373046875
    assert round(saving, 2) == g["value"]
    gb = saving * GOLD["double_quant_saving_65B_GB"]["params"] / 8 / 1e9
    assert round(gb) == GOLD["double_quant_saving_65B_GB"]["value"]


def test_full_finetune_memory_matches_page():
    g = GOLD["full_finetune_65B_GB"]
    assert accounting.full_finetune_bytes(g["params"]) / 1e9 == g["value"]


def test_lora_parameter_example():
    g = GOLD["lora_parameter_example"]
    assert g["A"] * g["B"] == g["full"]
    assert accounting.lora_params(g["A"], g["B"], g["r"]) == g["lora"]


def test_lora_7b_rank8_size():
    g = GOLD["lora_7B_r8_MB"]
    layers, hidden, _ = accounting.LLAMA["7B"]
    mb = accounting.lora_qv_bytes(layers, hidden, g["r"]) / 1e6
    assert round(mb) == g["value"]


def test_full65b_resident_size():
    g = WORKLOAD["full65b_resident_GB"]
    params = accounting.linear_params(*accounting.LLAMA["65B"])
    total = 0
    for (n, k) in [(8192, 8192)] * 4 + [(22016, 8192)] * 2 + [(8192, 22016)]:
        total += nf4.storage_bytes(n * k)
    total *= 80
    assert params == 64_760_053_760
    assert abs(total / 1e9 - g["value"]) < 1.0


@pytest.mark.parametrize("other", ["int4_k7", "int4_k8", "fp4"])
def test_nf4_has_lower_error_than_int4_and_fp4(other):
    w = np.random.Generator(np.random.PCG64(11)).normal(0, 0.02, 1 << 18).astype(np.float32)
    assert baselines.mse(w, "nf4") < baselines.mse(w, other)


def test_double_quant_does_not_degrade():
    w = np.random.Generator(np.random.PCG64(12)).normal(0, 0.02, 1 << 18).astype(np.float32)
    a, b = baselines.mse(w, "nf4"), baselines.mse(w, "nf4_dq")
    assert abs(b - a) / a < 0.01


def test_comparison_levels():
    assert baselines.int4_levels("k7").size == 15
    assert baselines.fp4_levels().size == 15 and baselines.fp4_levels().max() == 1.0
