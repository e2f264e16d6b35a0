"""Host checks of the bf16 input conversions that the parity tests rely on:
rounding fp32 draws to bf16 words and widening bf16 words back to fp32."""

import numpy as np
import pytest

from bit_nf4_quantized_21_amd import synth

torch = pytest.importorskip("torch")


def test_widening_known_words():
    bits = np.array([0x3F80, 0xC000, 0x3C80, 0x0000, 0x8000, 0x0001, 0x7F7F, 0x7F80], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -6, 0.0, -0.0, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, np.inf]
    got = synth.from_bf16_bits(bits)
    assert got.dtype == np.float32
    assert [float(x) for x in got] == want
    assert np.signbit(got[4]) and not np.signbit(got[3])


def test_widening_matches_torch_on_every_word():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = synth.from_bf16_bits(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    finite = ~np.isnan(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.isnan(got[~finite]).all()


def test_rounding_then_widening_is_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -0.02], dtype=np.float32)
    back = synth.from_bf16_bits(synth.to_bf16_bits(x))
    # 8 significant bits: the halfway points go to the even neighbour
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2.0 ** -6 and back[3] == 1.0 + 2.0 ** -7
    assert abs(back[4] - np.float32(-0.02)) <= 2.0 ** -6 * 2.0 ** -8 * 0.5
