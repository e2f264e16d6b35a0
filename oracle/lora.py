"""Forward and backward of the frozen NF4 linear layer with a LoRA adapter, in
fp64.  TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * QLoRA backpropagates through a frozen 4-bit base model into low-rank
    adapters ("QLoRA: Efficient Finetuning of Quantized LLMs", fugumt.com,
    Abstract): the base weight gets no gradient, the adapters do.
  * The LoRA tutorial (szsimon.cn), section on the weight update: the output
    is h = W x + dW x with dW = W_A W_B, W_A of size A x r and W_B of size
    r x B; W stays frozen and only W_A and W_B are trained; a scale alpha
    multiplies the adapter output (section on the rank and alpha).

Readings:
  R7  Row-vector convention with tokens as rows: X [T,K], dequantized weight
      W' [N,K], adapter A [K,r] and B [r,N], scale s = alpha / r (computed in
      fp32, exact in every configuration used here):
          Y = X W'^T + s (X A) B.
      In the tutorial's notation A plays W_B^T and B plays W_A^T.
  R8  With upstream gradient dY [T,N] and G = dY B^T [T,r]:
          dX = dY W' + s G A^T,   dA = s X^T G,   dB = s (X A)^T dY,
      and no gradient for the frozen W.  These follow from Y being linear
      in X, in A and in B.
All products are evaluated in fp64 from the exact values of the bf16 inputs
(and the bf16-rounded dequantized weight), with no intermediate rounding.
"""

from __future__ import annotations

import numpy as np


def lora_scale(alpha: float, r: int) -> float:
    """s = alpha / r computed in fp32 (the library computes it the same way)."""
    return float(np.float32(alpha) / np.float32(r))


def linear_fwd(X, Wd, A, B, alpha: float, r: int):
    """R7.  Returns (Y [T,N], XA [T,r]) in fp64."""
    X = np.asarray(X, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    s = lora_scale(alpha, r)
    XA = X @ A
    Y = X @ Wd.T + s * (XA @ B)
    return Y, XA


def linear_bwd(dY, X, Wd, A, B, alpha: float, r: int):
    """R8.  Returns (dX [T,K], dA [K,r], dB [r,N], G [T,r]) in fp64."""
    dY = np.asarray(dY, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    s = lora_scale(alpha, r)
    G = dY @ B.T
    dX = dY @ Wd + s * (G @ A.T)
    dA = s * (X.T @ G)
    dB = s * ((X @ A).T @ dY)
    return dX, dA, dB, G


def linear_fwd_rows(X_rows, Wd, A, B, alpha: float, r: int):
    """Forward for a subset of token rows (the rows are independent)."""
    return linear_fwd(X_rows, Wd, A, B, alpha, r)


def dx_rows(dY_rows, Wd, A, B, alpha: float, r: int):
    """dX for a subset of token rows (rows of dX depend only on rows of dY)."""
    dY_rows = np.asarray(dY_rows, dtype=np.float64)
    s = lora_scale(alpha, r)
    G = dY_rows @ np.asarray(B, dtype=np.float64).T
    return dY_rows @ np.asarray(Wd, dtype=np.float64) + s * (G @ np.asarray(A, dtype=np.float64).T)


def adapter_grads(dY, X, A, B, alpha: float, r: int):
    """R8 for the adapter alone: (dA [K,r], dB [r,N], G [T,r]) in fp64, the
    same products as linear_bwd without dX (which needs the whole base
    weight)."""
    dY = np.asarray(dY, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    s = lora_scale(alpha, r)
    G = dY @ B.T
    dA = s * (X.T @ G)
    dB = s * ((X @ A).T @ dY)
    return dA, dB, G
