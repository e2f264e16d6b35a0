"""Pins for the layer algebra (readings R7, R8): brute-force loops on tiny
shapes, finite differences of the linear loss, LoRA identities from the
tutorial page (dW = 0 when W_B = 0; merged weight W' = W + W_A W_B)."""

import numpy as np
import pytest

from oracle import lora, nf4


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _tiny(seed=0, T=3, K=128, N=5, r=2):
    rng = _rng(seed)
    X = nf4.bf16_round(rng.normal(0, 1, (T, K)).astype(np.float32))
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    codes, q8, s2, _ = nf4.quantize_all(W)
    Wd = nf4.dequantize(codes, q8, s2, W.size, "bf16").reshape(N, K)
    A = nf4.bf16_round(rng.uniform(-1 / np.sqrt(K), 1 / np.sqrt(K), (K, r)).astype(np.float32))
    B = nf4.bf16_round(rng.normal(0, 0.01, (r, N)).astype(np.float32))
    dY = nf4.bf16_round(rng.normal(0, 1, (T, N)).astype(np.float32))
    return X, Wd, A, B, dY


def _loops_fwd(X, Wd, A, B, s):
    T, K = X.shape
    N, r = Wd.shape[0], A.shape[1]
    Y = [[0.0] * N for _ in range(T)]
    XA = [[0.0] * r for _ in range(T)]
    for t in range(T):
        for j in range(r):
            XA[t][j] = sum(float(X[t, k]) * float(A[k, j]) for k in range(K))
        for n in range(N):
            base = sum(float(X[t, k]) * float(Wd[n, k]) for k in range(K))
            low = sum(XA[t][j] * float(B[j, n]) for j in range(r))
            Y[t][n] = base + s * low
    return np.array(Y), np.array(XA)


def _loops_bwd(dY, X, Wd, A, B, s):
    T, K = X.shape
    N, r = Wd.shape[0], A.shape[1]
    G = [[sum(float(dY[t, n]) * float(B[j, n]) for n in range(N)) for j in range(r)] for t in range(T)]
    XA = [[sum(float(X[t, k]) * float(A[k, j]) for k in range(K)) for j in range(r)] for t in range(T)]
    dX = [[sum(float(dY[t, n]) * float(Wd[n, k]) for n in range(N)) + s * sum(G[t][j] * float(A[k, j]) for j in range(r))
           for k in range(K)] for t in range(T)]
    dA = [[s * sum(float(X[t, k]) * G[t][j] for t in range(T)) for j in range(r)] for k in range(K)]
    dB = [[s * sum(XA[t][j] * float(dY[t, n]) for t in range(T)) for n in range(N)] for j in range(r)]
    return np.array(dX), np.array(dA), np.array(dB)


@pytest.mark.parametrize("alpha,r", [(16.0, 2), (16.0, 8), (1.0, 4)])
def test_forward_matches_loops(alpha, r):
    X, Wd, A, B, _ = _tiny(1, r=r)
    s = lora.lora_scale(alpha, r)
    Y, XA = lora.linear_fwd(X, Wd, A, B, alpha, r)
    Yl, XAl = _loops_fwd(X, Wd, A, B, s)
    assert np.allclose(Y, Yl, rtol=1e-12, atol=1e-13)
    assert np.allclose(XA, XAl, rtol=1e-12, atol=1e-13)


def test_backward_matches_loops():
    X, Wd, A, B, dY = _tiny(2, T=4, K=64, N=6, r=3)
    s = lora.lora_scale(16.0, 3)
    dX, dA, dB, _ = lora.linear_bwd(dY, X, Wd, A, B, 16.0, 3)
    ldX, ldA, ldB = _loops_bwd(dY, X, Wd, A, B, s)
    assert np.allclose(dX, ldX, rtol=1e-12, atol=1e-13)
    assert np.allclose(dA, ldA, rtol=1e-12, atol=1e-13)
    assert np.allclose(dB, ldB, rtol=1e-12, atol=1e-13)


def test_adapter_grads_match_loops():
    """adapter_grads (the dA, dB used at full layer sizes) against the triple
    loops, including the intermediate G = dY B^T."""
    X, Wd, A, B, dY = _tiny(4, T=5, K=64, N=6, r=3)
    s = lora.lora_scale(16.0, 3)
    dA, dB, G = lora.adapter_grads(dY, X, A, B, 16.0, 3)
    _, ldA, ldB = _loops_bwd(dY, X, Wd, A, B, s)
    lG = np.array([[sum(dY[t, n] * B[j, n] for n in range(6)) for j in range(3)] for t in range(5)])
    assert np.allclose(dA, ldA, rtol=1e-12, atol=1e-13)
    assert np.allclose(dB, ldB, rtol=1e-12, atol=1e-13)
    assert np.allclose(G, lG, rtol=1e-12, atol=1e-13)


def test_gradients_by_central_differences():
    """L = <dY, Y> is linear in X, in A and in B separately, so a central
    difference along any direction equals the gradient's inner product with
    that direction up to rounding."""
    X, Wd, A, B, dY = _tiny(3, T=4, K=64, N=7, r=4)
    alpha, r = 16.0, 4
    dX, dA, dB, _ = lora.linear_bwd(dY, X, Wd, A, B, alpha, r)
    L = lambda X_, A_, B_: float(np.sum(dY * lora.linear_fwd(X_, Wd, A_, B_, alpha, r)[0]))
    rng = _rng(30)
    for _ in range(3):
        EX, EA, EB = rng.normal(size=X.shape), rng.normal(size=A.shape), rng.normal(size=B.shape)
        h = 0.5
        assert np.isclose((L(X + h * EX, A, B) - L(X - h * EX, A, B)) / (2 * h), np.sum(dX * EX), rtol=1e-9)
        assert np.isclose((L(X, A + h * EA, B) - L(X, A - h * EA, B)) / (2 * h), np.sum(dA * EA), rtol=1e-9)
        assert np.isclose((L(X, A, B + h * EB) - L(X, A, B - h * EB)) / (2 * h), np.sum(dB * EB), rtol=1e-9)


def test_zero_up_projection_means_no_update():
    """W_B = 0 at initialisation makes dW = 0 (tutorial, rank-and-alpha
    section): Y is the base layer's output and A gets no gradient."""
    X, Wd, A, B, dY = _tiny(4)
    B0 = np.zeros_like(B)
    Y, _ = lora.linear_fwd(X, Wd, A, B0, 16.0, 2)
    assert np.array_equal(Y, X.astype(np.float64) @ Wd.astype(np.float64).T)
    _, dA, _, _ = lora.linear_bwd(dY, X, Wd, A, B0, 16.0, 2)
    assert np.all(dA == 0)


def test_zero_weight_isolates_adapter():
    X, _, A, B, _ = _tiny(5)
    W = np.zeros((5, 128), dtype=np.float32)
    codes, q8, s2, _ = nf4.quantize_all(W)
    Wd = nf4.dequantize(codes, q8, s2, W.size, "bf16").reshape(5, 128)
    assert np.all(Wd == 0)
    Y, XA = lora.linear_fwd(X, Wd, A, B, 16.0, 2)
    assert np.allclose(Y, 8.0 * (XA @ B.astype(np.float64)), rtol=1e-14, atol=0)


def test_merge_identity():
    """Tutorial, reducing-inference-overhead section: W' = W + W_A W_B gives
    the same output as keeping the factors separate."""
    X, Wd, A, B, _ = _tiny(6)
    s = lora.lora_scale(16.0, 2)
    Y, _ = lora.linear_fwd(X, Wd, A, B, 16.0, 2)
    merged = Wd.astype(np.float64) + s * (A.astype(np.float64) @ B.astype(np.float64)).T
    assert np.allclose(Y, X.astype(np.float64) @ merged.T, rtol=1e-12, atol=1e-13)


def test_scale_values():
    assert lora.lora_scale(16.0, 8) == 2.0 and lora.lora_scale(16.0, 64) == 0.25


@pytest.mark.parametrize("rows", [[0, 2, 3], [1], [3, 0]])
def test_dx_rows_matches_loops_and_full_backward(rows):
    """dx_rows (the dX reference for sampled token rows at full layer sizes)
    equals the triple-loop dX and linear_bwd's dX on those rows, so a dropped
    scale or a transposed factor in it would fail here."""
    X, Wd, A, B, dY = _tiny(7, T=4, K=64, N=6, r=3)
    alpha, r = 16.0, 3
    s = lora.lora_scale(alpha, r)
    got = lora.dx_rows(dY[rows], Wd, A, B, alpha, r)
    dX, _, _, _ = lora.linear_bwd(dY, X, Wd, A, B, alpha, r)
    ldX, _, _ = _loops_bwd(dY, X, Wd, A, B, s)
    assert np.allclose(got, dX[rows], rtol=1e-13, atol=1e-14)
    assert np.allclose(got, ldX[rows], rtol=1e-12, atol=1e-13)
    # the adapter part alone carries the scale: with W' = 0 only s G A^T remains
    got0 = lora.dx_rows(dY[rows], np.zeros_like(Wd), A, B, alpha, r)
    G = dY[rows].astype(np.float64) @ B.astype(np.float64).T
    assert np.allclose(got0, s * (G @ A.astype(np.float64).T), rtol=1e-13, atol=1e-15)
    assert not np.allclose(got0, G @ A.astype(np.float64).T, rtol=1e-3)


def test_forward_rows_match_full_forward():
    """linear_fwd_rows on a subset of tokens equals those rows of the whole
    forward (rows of Y and XA depend only on the same rows of X)."""
    X, Wd, A, B, _ = _tiny(8, T=5)
    Y, XA = lora.linear_fwd(X, Wd, A, B, 16.0, 2)
    Yr, XAr = lora.linear_fwd_rows(X[[4, 1]], Wd, A, B, 16.0, 2)
    assert np.array_equal(Yr, Y[[4, 1]]) and np.array_equal(XAr, XA[[4, 1]])
