"""The tolerance rule must accept a correctly rounded result and reject the
plausible mistakes (a dropped LoRA term, a transposed operand, a wrong sign)."""

import numpy as np

from oracle import compare, lora, nf4


def _case(seed=0, T=64, K=256, N=96, r=8):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = nf4.bf16_round(rng.normal(0, 1, (T, K)).astype(np.float32))
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    codes, q8, s2, _ = nf4.quantize_all(W)
    Wd = nf4.dequantize(codes, q8, s2, W.size, "bf16").reshape(N, K)
    A = nf4.bf16_round(rng.uniform(-1 / 16, 1 / 16, (K, r)).astype(np.float32))
    B = nf4.bf16_round(rng.normal(0, 0.05, (r, N)).astype(np.float32))
    return X, Wd, A, B


def test_bf16_rounded_exact_result_passes():
    X, Wd, A, B = _case()
    Y, _ = lora.linear_fwd(X, Wd, A, B, 16.0, 8)
    got = nf4.bf16_round(Y.astype(np.float32))
    ok, info = compare.check_close(got, Y)
    assert ok, info


def test_mistakes_fail():
    X, Wd, A, B = _case(1)
    Y, XA = lora.linear_fwd(X, Wd, A, B, 16.0, 8)
    no_lora = X.astype(np.float64) @ Wd.astype(np.float64).T
    assert not compare.check_close(no_lora, Y)[0]
    wrong_sign = no_lora - 2.0 * (XA @ B.astype(np.float64))
    assert not compare.check_close(wrong_sign, Y)[0]
    perm = Y[:, ::-1]
    assert not compare.check_close(perm, Y)[0]
    assert not compare.check_close(Y[:-1], Y)[0]


def test_ulp():
    assert compare.ulp_bf16(np.array([1.0]))[0] == 2 ** -7
    assert compare.ulp_bf16(np.array([3.0]))[0] == 2 ** -6
    assert compare.ulp_bf16(np.array([0.0]))[0] == 0.0
