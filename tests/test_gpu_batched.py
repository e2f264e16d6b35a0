"""GPU parity of the grouped forward and backward on the GEMM path, where
runs of same-shape linears share one dequant-GEMM launch: every linear's Y,
dX against the oracle (bf16 tolerance) and against its own single call
(the contraction may be sliced differently, so within tolerance); XA, dA and
dB within rounding of the single call (the rank-r contractions are chunked
for the whole batch); mixed-shape runs; T = 0; and the full-size 65B q/k/v
batch on sampled token rows."""

import numpy as np
import pytest

from bit_nf4_quantized_21_amd import synth
from oracle import compare, lora, nf4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _q():
    from bit_nf4_quantized_21_amd import qlora
    return qlora


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _make(shapes, T, r, seed0):
    q = _q()
    out = []
    for i, (N, K) in enumerate(shapes):
        seed = seed0 + i
        W = torch.from_numpy(synth.weight(N, K, seed).ravel()).cuda()
        codes, q8, s2 = q.quantize_dq(W)
        out.append(dict(N=N, K=K, seed=seed, codes=codes, q8=q8, s2=s2,
                        X=_bf16_dev(synth.x_bits(T, K, seed)), A=_bf16_dev(synth.a_bits(K, r, seed)),
                        B=_bf16_dev(synth.b_bits(r, N, seed)), dY=_bf16_dev(synth.dy_bits(T, N, seed))))
    return out


def _oracle(L, T, r, alpha, rows=None):
    N, K, seed = L["N"], L["K"], L["seed"]
    codes, q8, s2, _ = nf4.quantize_all(synth.weight(N, K, seed))
    Wd = nf4.dequantize(codes, q8, s2, N * K, "bf16").reshape(N, K)
    X = nf4.bf16_bits_to_f32(synth.x_bits(T, K, seed))
    A = nf4.bf16_bits_to_f32(synth.a_bits(K, r, seed))
    B = nf4.bf16_bits_to_f32(synth.b_bits(r, N, seed))
    dY = nf4.bf16_bits_to_f32(synth.dy_bits(T, N, seed))
    rows = np.arange(T) if rows is None else rows
    Yr, _ = lora.linear_fwd(X[rows], Wd, A, B, alpha, r)
    dXr = lora.dx_rows(dY[rows], Wd, A, B, alpha, r)
    dAr, dBr, _ = lora.adapter_grads(dY, X, A, B, alpha, r)
    return Yr, dXr, dAr, dBr


def _close(name, got, ref):
    ok, info = compare.check_close(got, ref)
    assert ok, f"{name}: {info}"


@pytest.mark.parametrize("shapes,T,r", [
    ([(2048, 2048)] * 3, 300, 64),                            # one run of 3 (split tiles)
    ([(520, 640)] * 2 + [(776, 1024)] + [(520, 640)], 257, 16),  # runs 2, 1, 1; ragged
    ([(1024, 4096)] * 4 + [(1024, 4096)], 64, 8),             # a full run of 4, then 1
    ([(1024, 1024)] * 2, 200, 128),                           # two rank blocks, token chunks
    ([(1024, 2048)] * 3, 64, 72),                             # rank padded to 128, one token chunk
])
def test_grouped_gemm_path_against_oracle_and_single(shapes, T, r):
    print(f"batched {shapes} T={T} r={r}", flush=True)
    q = _q()
    alpha = 16.0
    Ls = _make(shapes, T, r, seed0=T + r)
    fo = q.linear_fwd_grouped(Ls, alpha, T, r)
    for L, (Y, XA) in zip(Ls, fo):
        L["XA"] = XA
    bo = q.linear_bwd_grouped(Ls, alpha, T, r)
    torch.cuda.synchronize()
    for L, (Y, XA), (dX, dA, dB) in zip(Ls, fo, bo):
        Y1, XA1 = q.linear_fwd(L["X"], L["codes"], L["q8"], L["s2"], L["A"], L["B"], alpha, L["N"])
        dX1, dA1, dB1 = q.linear_bwd(L["dY"], L["X"], XA1, L["codes"], L["q8"], L["s2"], L["A"], L["B"], alpha)
        torch.cuda.synchronize()
        # A batch cuts the rank-r contractions into chunks sized for the
        # whole batch, so its fp32 summation order (and the last bits) may
        # differ from a single launch's; both are checked against the oracle.
        xa_scale = float(XA1.abs().max())
        assert torch.allclose(XA, XA1, rtol=1e-5, atol=1e-6 * xa_scale)
        _close("dA vs single", _f64(dA), _f64(dA1))
        _close("dB vs single", _f64(dB), _f64(dB1))
        Yr, dXr, dAr, dBr = _oracle(L, T, r, alpha)
        _close("Y", _f64(Y), Yr)
        _close("dX", _f64(dX), dXr)
        _close("dA", _f64(dA), dAr)
        _close("dB", _f64(dB), dBr)
        _close("Y vs single", _f64(Y), _f64(Y1))
        _close("dX vs single", _f64(dX), _f64(dX1))


def test_grouped_backward_no_tokens_zeroes_adapter_grads():
    q = _q()
    Ls = _make([(512, 512)] * 2, 0, 8, seed0=5)
    for L in Ls:
        L["X"] = torch.empty(0, 512, dtype=torch.bfloat16, device="cuda")
        L["dY"] = torch.empty(0, 512, dtype=torch.bfloat16, device="cuda")
        L["XA"] = torch.empty(0, 8, dtype=torch.float32, device="cuda")
        L["dA"] = torch.full((512, 8), 1.0, dtype=torch.bfloat16, device="cuda")
        L["dB"] = torch.full((8, 512), 1.0, dtype=torch.bfloat16, device="cuda")
    out = q.linear_bwd_grouped(Ls, 16.0, 0, 8)
    torch.cuda.synchronize()
    for (_, dA, dB) in out:
        assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0


def test_grouped_65b_qkv_full_size_sampled_rows():
    """q, k, v of the 65B set (8192 x 8192) at 512 tokens in one batched
    launch each way (192 whole-contraction tiles), sampled rows of Y and dX
    and all of dA, dB against the oracle."""
    print("batched 65b qkv", flush=True)
    q = _q()
    T, r, alpha = 512, 64, 16.0
    Ls = _make([(8192, 8192)] * 3, T, r, seed0=600)
    fo = q.linear_fwd_grouped(Ls, alpha, T, r)
    for L, (Y, XA) in zip(Ls, fo):
        L["XA"] = XA
    bo = q.linear_bwd_grouped(Ls, alpha, T, r)
    torch.cuda.synchronize()
    q.device_status()
    rows = np.array([0, 1, 255, 256, 300, 511])
    for L, (Y, _), (dX, dA, dB) in zip(Ls, fo, bo):
        Yr, dXr, dAr, dBr = _oracle(L, T, r, alpha, rows)
        _close("Y", _f64(Y)[rows], Yr)
        _close("dX", _f64(dX)[rows], dXr)
        _close("dA", _f64(dA), dAr)
        _close("dB", _f64(dB), dBr)


def test_grouped_gemm_path_deterministic():
    """The batched forward and backward twice on the same inputs (with other
    work between, so the split hand-offs finish in another order): Y, XA,
    dX, dA, dB identical bit for bit.  The reductions sum in a fixed order
    whatever the timing."""
    q = _q()
    T, r, alpha = 300, 64, 16.0
    Ls = _make([(2048, 2048)] * 3 + [(2048, 5632)], T, r, seed0=700)

    def run():
        fo = q.linear_fwd_grouped(Ls, alpha, T, r)
        for L, (Y, XA) in zip(Ls, fo):
            L["XA"] = XA
        bo = q.linear_bwd_grouped(Ls, alpha, T, r)
        torch.cuda.synchronize()
        return [t.clone() for pair in fo for t in pair] + [t.clone() for tri in bo for t in tri]

    a = run()
    junk = torch.randn(4096, 4096, device="cuda") @ torch.randn(4096, 4096, device="cuda")
    torch.cuda.synchronize()
    del junk
    b = run()
    q.device_status()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


def _random_cases(n, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        count = int(rng.integers(2, 5))
        N = int(rng.integers(1, 320)) * 8
        K = int(rng.integers(1, 40)) * 64
        T = int(rng.integers(17, 700))
        r = int(rng.choice([8, 16, 24, 64, 72, 120, 128]))
        cases.append(([(N, K)] * count, T, r))
    return cases


@pytest.mark.parametrize("shapes,T,r", _random_cases(6))
def test_batched_random_shapes_against_oracle(shapes, T, r):
    """Seeded random batches (2-4 same-shape linears, N and K up to ~2500,
    ragged T up to 700, ranks 8-128): every output against the oracle on
    sampled token rows (Y, dX) and in full (dA, dB)."""
    print(f"batched random {shapes[0]} x{len(shapes)} T={T} r={r}", flush=True)
    q = _q()
    alpha = 16.0
    Ls = _make(shapes, T, r, seed0=T * 7 + r)
    fo = q.linear_fwd_grouped(Ls, alpha, T, r)
    for L, (Y, XA) in zip(Ls, fo):
        L["XA"] = XA
    bo = q.linear_bwd_grouped(Ls, alpha, T, r)
    torch.cuda.synchronize()
    q.device_status()
    rows = np.unique(np.array([0, 1, T // 3, T // 2, T - 2, T - 1]))
    for L, (Y, _), (dX, dA, dB) in zip(Ls, fo, bo):
        Yr, dXr, dAr, dBr = _oracle(L, T, r, alpha, rows)
        _close("Y", _f64(Y)[rows], Yr)
        _close("dX", _f64(dX)[rows], dXr)
        _close("dA", _f64(dA), dAr)
        _close("dB", _f64(dB), dBr)
