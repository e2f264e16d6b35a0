"""GPU parity of quantization, double quantization and dequantization with the
oracle: bit-exact codes, absmax, q8, s2 and dequantized weights."""

import numpy as np
import pytest

from oracle import nf4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _q():
    from bit_nf4_quantized_21_amd import qlora
    return qlora


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _gpu_quant_all(w):
    q = _q()
    W = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32).ravel()).cuda()
    codes, absmax = q.quantize_nf4(W)
    q8, s2 = q.double_quant(absmax)
    torch.cuda.synchronize()
    return codes, absmax, q8, s2


@pytest.mark.parametrize("n", [2, 64, 130, 512 * 512, 64 * 1000 + 38, 4096 * 4096])
def test_quantize_bit_exact(n):
    w = _rng(n).normal(0, 0.02, n).astype(np.float32)
    print(f"quantize n={n}", flush=True)
    codes, absmax, q8, s2 = _gpu_quant_all(w)
    oc, oq8, os2, oa = nf4.quantize_all(w)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), oa.view(np.uint32))
    assert np.array_equal(q8.cpu().numpy(), oq8)
    assert np.array_equal(s2.cpu().numpy().view(np.uint32), os2.view(np.uint32))


def test_quantize_largest_linear_sampled_groups():
    """The largest linear of the 65B set (22016 x 8192, 180 M weights) in one
    call; 48 double-quant groups (256 blocks, 16384 weights each, so a group
    is self-contained) at random positions plus the first and the last are
    checked bit-exact against the oracle run on those groups alone."""
    N, K = 22016, 8192
    n = N * K
    print(f"quantize n={n}", flush=True)
    w = _rng(77).normal(0, 0.02, n).astype(np.float32)
    codes, absmax, q8, s2 = _gpu_quant_all(w)
    codes, absmax, q8, s2 = codes.cpu().numpy(), absmax.cpu().numpy(), q8.cpu().numpy(), s2.cpu().numpy()
    gsz = 64 * 256
    ng = n // gsz
    groups = np.concatenate([[0, ng - 1], _rng(78).choice(np.arange(1, ng - 1), 48, replace=False)])
    for g in groups:
        oc, oq8, os2, oa = nf4.quantize_all(w[g * gsz:(g + 1) * gsz])
        assert np.array_equal(codes[g * gsz // 2:(g + 1) * gsz // 2], oc), g
        assert np.array_equal(absmax[g * 256:(g + 1) * 256].view(np.uint32), oa.view(np.uint32)), g
        assert np.array_equal(q8[g * 256:(g + 1) * 256], oq8), g
        assert np.array_equal(s2[g:g + 1].view(np.uint32), os2.view(np.uint32)), g


def _gpu_quant_bf16(bits):
    q = _q()
    W = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    codes, absmax = q.quantize_nf4(W)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), absmax.cpu().numpy()


@pytest.mark.parametrize("n", [2, 64, 130, 64 * 1000 + 38, 4096 * 4096])
def test_quantize_bf16_weights_bit_exact(n):
    """bf16 weights: codes and absmax equal the oracle's on the values the
    bf16 words encode, and the fp32 entry point's on the same values."""
    from bit_nf4_quantized_21_amd import synth
    bits = synth.to_bf16_bits(_rng(n + 5).normal(0, 0.02, n))
    bits[:64] = 0                 # an all-zero block: code 7 throughout
    bits[64:128:2] = 0x8000       # negative zeros inside a block
    print(f"quantize bf16 n={n}", flush=True)
    codes, absmax = _gpu_quant_bf16(bits)
    w = synth.from_bf16_bits(bits)
    oc, _, _, oa = nf4.quantize_all(w)
    assert np.array_equal(codes, oc)
    assert np.array_equal(absmax.view(np.uint32), oa.view(np.uint32))
    fc, fa, _, _ = _gpu_quant_all(w)
    assert np.array_equal(codes, fc.cpu().numpy())
    assert np.array_equal(absmax.view(np.uint32), fa.cpu().numpy().view(np.uint32))


def test_quantize_bf16_mlp_weight_sampled_groups():
    """An 11008 x 4096 bf16 weight (45 M weights) in one call; 40 groups of
    16384 weights at random positions plus the first and the last checked
    bit-exact against the oracle run on those groups alone."""
    from bit_nf4_quantized_21_amd import synth
    N, K = 11008, 4096
    n = N * K
    print(f"quantize bf16 n={n}", flush=True)
    bits = synth.to_bf16_bits(_rng(79).normal(0, 0.02, n))
    codes, absmax = _gpu_quant_bf16(bits)
    gsz = 64 * 256
    ng = n // gsz
    groups = np.concatenate([[0, ng - 1], _rng(80).choice(np.arange(1, ng - 1), 40, replace=False)])
    for g in groups:
        oc, _, _, oa = nf4.quantize_all(synth.from_bf16_bits(bits[g * gsz:(g + 1) * gsz]))
        assert np.array_equal(codes[g * gsz // 2:(g + 1) * gsz // 2], oc), g
        assert np.array_equal(absmax[g * 256:(g + 1) * 256].view(np.uint32), oa.view(np.uint32)), g


def test_quantize_specials_and_ties():
    m = nf4.midpoints()
    rep = [j for j in range(15) if float(np.float32(m[j])) == m[j]]
    blk = np.zeros(64 * 4, dtype=np.float32)
    blk[0], blk[1] = 1.0, -1.0
    for i, j in enumerate(rep):
        blk[3 + 2 * i] = np.float32(m[j])
        blk[4 + 2 * i] = np.nextafter(np.float32(m[j]), np.float32(2.0))
    blk[64:128] = 0.0                                   # all-zero block -> code 7
    blk[128:192] = _rng(1).normal(0, 1e-30, 64)        # tiny values
    blk[192:256] = _rng(2).normal(0, 100.0, 64)
    codes, absmax, q8, s2 = _gpu_quant_all(blk)
    oc, oq8, os2, oa = nf4.quantize_all(blk)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(absmax.cpu().numpy(), oa)
    assert np.array_equal(q8.cpu().numpy(), oq8)
    assert np.array_equal(s2.cpu().numpy(), os2)


def test_double_quant_ties_bit_exact():
    q = _q()
    ties = np.array([255.0] + [k + 0.5 for k in range(254)] + [3.0], dtype=np.float32)
    rest = np.abs(_rng(3).normal(0, 0.02, 300)).astype(np.float32)
    a = np.concatenate([ties, rest])
    q8, s2 = q.double_quant(torch.from_numpy(a).cuda())
    oq8, os2 = nf4.double_quant(a)
    assert np.array_equal(q8.cpu().numpy(), oq8)
    assert np.array_equal(s2.cpu().numpy(), os2)


@pytest.mark.parametrize("n", [64, 200, 512 * 512, 64 * 777 + 10])
@pytest.mark.parametrize("bf16", [True, False])
def test_dequantize_bit_exact(n, bf16):
    q = _q()
    w = _rng(n + 7).normal(0, 0.02, n).astype(np.float32)
    codes, absmax, q8, s2 = _gpu_quant_all(w)
    out = q.dequantize_nf4(codes, q8, s2, n, dtype=torch.bfloat16 if bf16 else torch.float32)
    torch.cuda.synchronize()
    ref = nf4.dequantize(codes.cpu().numpy(), q8.cpu().numpy(), s2.cpu().numpy(), n, "bf16" if bf16 else "f32")
    got = out.float().cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_deterministic_repeat():
    w = _rng(9).normal(0, 0.02, 1 << 20).astype(np.float32)
    a = _gpu_quant_all(w)
    b = _gpu_quant_all(w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
