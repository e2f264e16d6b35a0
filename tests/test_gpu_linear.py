"""GPU parity of the forward and backward pass with the fp64 oracle.

Bar: bit-exact NF4 codes and constants; for bf16 outputs and gradients a
relative Frobenius error <= 5e-3 and an elementwise error <= 1e-2 of the
output RMS (plus half a bf16 ulp, reading R10).  XA (fp32 output) must match
to fp32 accumulation accuracy.  Inputs come from the seeded generator; the
oracle quantizes W itself.  At full layer sizes, Y and dX are checked on
sampled token rows (rows are independent) and dA, dB in full.
"""

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


def _f32(t):
    return t.float().cpu().numpy().astype(np.float64)


class Case:
    def __init__(self, N, K, T, r, alpha=16.0, seed=0):
        self.N, self.K, self.T, self.r, self.alpha = N, K, T, r, alpha
        self.W = synth.weight(N, K, seed)
        self.Xb = synth.x_bits(T, K, seed)
        self.Ab = synth.a_bits(K, r, seed)
        self.Bb = synth.b_bits(r, N, seed)
        self.dYb = synth.dy_bits(T, N, seed)
        self.X = nf4.bf16_bits_to_f32(self.Xb)
        self.A = nf4.bf16_bits_to_f32(self.Ab)
        self.B = nf4.bf16_bits_to_f32(self.Bb)
        self.dY = nf4.bf16_bits_to_f32(self.dYb)

    def oracle_weight(self):
        codes, q8, s2, _ = nf4.quantize_all(self.W)
        Wd = nf4.dequantize(codes, q8, s2, self.N * self.K, "bf16").reshape(self.N, self.K)
        return codes, q8, s2, Wd

    def gpu(self, bwd=True):
        q = _q()
        Wg = torch.from_numpy(self.W.ravel()).cuda()
        codes, absmax = q.quantize_nf4(Wg)
        q8, s2 = q.double_quant(absmax)
        del Wg
        Xg, Ag, Bg = _bf16_dev(self.Xb), _bf16_dev(self.Ab), _bf16_dev(self.Bb)
        Y, XA = q.linear_fwd(Xg, codes, q8, s2, Ag, Bg, self.alpha, self.N)
        out = {"codes": codes, "q8": q8, "s2": s2, "Y": Y, "XA": XA}
        if bwd:
            dYg = _bf16_dev(self.dYb)
            dX, dA, dB = q.linear_bwd(dYg, Xg, XA, codes, q8, s2, Ag, Bg, self.alpha)
            out.update(dX=dX, dA=dA, dB=dB)
        torch.cuda.synchronize()
        return out


def _assert_close(name, got, ref):
    ok, info = compare.check_close(got, ref)
    assert ok, f"{name}: {info}"


def _check_xa(XA, X, A, ref):
    """XA = X A in fp32 from exact bf16 products: every element within the
    first-order bound of K-term fp32 summation in any order,
    |got - ref| <= 2 K u sum_k |X_tk A_kj| (u = 2^-24), plus the rounding of
    the stored fp32 value."""
    K = X.shape[1]
    mag = np.abs(np.asarray(X, np.float64)) @ np.abs(np.asarray(A, np.float64))
    bound = 2 * K * 2.0 ** -24 * mag + 2.0 ** -24 * np.abs(ref) + 1e-38
    err = np.abs(XA - ref)
    assert np.all(err <= bound), float(np.max(err / bound))
    assert compare.rel_fro(XA, ref) < 1e-5


def _check(case, out, rows=None, bwd=True):
    codes, q8, s2, Wd = case.oracle_weight()
    assert np.array_equal(out["codes"].cpu().numpy(), codes)
    assert np.array_equal(out["q8"].cpu().numpy(), q8)
    assert np.array_equal(out["s2"].cpu().numpy(), s2)
    rows = np.arange(case.T) if rows is None else rows
    Yref, XAref = lora.linear_fwd(case.X[rows], Wd, case.A, case.B, case.alpha, case.r)
    _assert_close("Y", _f32(out["Y"])[rows], Yref)
    XA = out["XA"].cpu().numpy().astype(np.float64)[rows]
    _check_xa(XA, case.X[rows], case.A, XAref)
    if not bwd:
        return
    dXref = lora.dx_rows(case.dY[rows], Wd, case.A, case.B, case.alpha, case.r)
    _assert_close("dX", _f32(out["dX"])[rows], dXref)
    dAref, dBref, _ = lora.adapter_grads(case.dY, case.X, case.A, case.B, case.alpha, case.r)
    _assert_close("dA", _f32(out["dA"]), dAref)
    _assert_close("dB", _f32(out["dB"]), dBref)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_gemv_path_small_tokens(T):
    print(f"gemv T={T}", flush=True)
    c = Case(512, 512, T, 8, seed=10 + T)
    _check(c, c.gpu())


@pytest.mark.parametrize("N,K,T,r", [(1000, 11008, 3, 128), (24, 64, 16, 8), (4104, 2048, 9, 72),
                                     (776, 8192, 2, 64)])
def test_gemv_path_ragged(N, K, T, r):
    """GEMV path with N not a multiple of 16, one to 32 XA producers (last
    slice short), adapter ranks 8, 64, 72 and 128."""
    print(f"gemv ragged N={N} K={K} T={T} r={r}", flush=True)
    c = Case(N, K, T, r, seed=N + K + T + r)
    _check(c, c.gpu(bwd=False), bwd=False)


def test_gemv_path_repeated_calls_identical():
    """More back-to-back GEMV-path calls than there are hand-off records, two
    shapes interleaved: every call returns exactly the first call's result."""
    print("gemv repeat", flush=True)
    q = _q()
    outs = []
    for (N, K, T, r, seed) in [(512, 1024, 4, 16, 21), (272, 4096, 7, 128, 22)]:
        c = Case(N, K, T, r, seed=seed)
        Wg = torch.from_numpy(c.W.ravel()).cuda()
        codes, absmax = q.quantize_nf4(Wg)
        q8, s2 = q.double_quant(absmax)
        outs.append((c, codes, q8, s2, _bf16_dev(c.Xb), _bf16_dev(c.Ab), _bf16_dev(c.Bb)))
    first = []
    for (c, codes, q8, s2, Xg, Ag, Bg) in outs:
        first.append(q.linear_fwd(Xg, codes, q8, s2, Ag, Bg, c.alpha, c.N))
    torch.cuda.synchronize()
    for it in range(150):
        i = it % 2
        c, codes, q8, s2, Xg, Ag, Bg = outs[i]
        Y, XA = q.linear_fwd(Xg, codes, q8, s2, Ag, Bg, c.alpha, c.N)
        assert torch.equal(Y, first[i][0]) and torch.equal(XA, first[i][1]), it
    c = outs[1][0]
    Wd = c.oracle_weight()[3]
    Yref, _ = lora.linear_fwd(c.X, Wd, c.A, c.B, c.alpha, c.r)
    _assert_close("Y", _f32(first[1][0]), Yref)


def test_tiny_config_fwd_bwd():
    """W 512x512, X 32x512, r=8, alpha=16: the small workload in full."""
    print("tiny", flush=True)
    c = Case(512, 512, 32, 8, seed=0)
    _check(c, c.gpu())


@pytest.mark.parametrize("N,K,T,r", [(520, 576, 17, 16), (776, 640, 257, 64), (264, 1088, 300, 24),
                                     (1024, 512, 513, 128)])
def test_gemm_path_ragged(N, K, T, r):
    """Several tiles in every dimension with ragged tails (N not a multiple of
    256, K % 128 == 64, T not a multiple of 256), several ranks."""
    print(f"ragged N={N} K={K} T={T} r={r}", flush=True)
    c = Case(N, K, T, r, seed=N + K + T)
    _check(c, c.gpu())


def test_gemv_config_llama7b_qproj():
    """4096x4096 q_proj, T=4, r=64: the HBM-bound small-token path in full."""
    print("gemv 7B q_proj", flush=True)
    c = Case(4096, 4096, 4, 64, seed=1)
    _check(c, c.gpu(bwd=False), bwd=False)


@pytest.mark.parametrize("N,K", [(11008, 4096), (4096, 11008)])
def test_llama7b_mlp_full_size_sampled(N, K):
    """7B MLP linears at T=2048: Y and dX on 48 sampled rows, dA and dB in full."""
    print(f"7B MLP N={N} K={K}", flush=True)
    c = Case(N, K, 2048, 64, seed=N)
    out = c.gpu()
    rows = np.random.Generator(np.random.PCG64(7)).choice(2048, 48, replace=False)
    rows = np.sort(np.concatenate([rows, [0, 2047]]))
    _check(c, out, rows=rows)


@pytest.mark.parametrize("N,K,T", [(6656, 6656, 4096), (17920, 6656, 4096), (6656, 17920, 4096),
                                   (8192, 8192, 512), (22016, 8192, 512), (8192, 22016, 512)])
def test_33b_65b_linears_full_size_sampled(N, K, T):
    """The 33B layer's linears at T=4096 and the 65B set's at T=512 (r=64,
    alpha=16): Y and dX on 40 sampled rows, dA and dB in full."""
    print(f"full size N={N} K={K} T={T}", flush=True)
    c = Case(N, K, T, 64, seed=N + 3 * K + T)
    out = c.gpu()
    rows = np.random.Generator(np.random.PCG64(11)).choice(T, 38, replace=False)
    rows = np.sort(np.concatenate([rows, [0, T - 1]]))
    _check(c, out, rows=rows)


def test_three_slice_split_tiles():
    """72 tiles of 256 x 256 (9 per XCD) in both GEMMs: the last round cuts
    every tile into three contraction slices, so the combine adds two other
    slices' partials in slice order."""
    print("three-slice split", flush=True)
    c = Case(2304, 2304, 2048, 16, seed=23)
    out = c.gpu()
    rows = np.random.Generator(np.random.PCG64(5)).choice(2048, 30, replace=False)
    rows = np.sort(np.concatenate([rows, [0, 255, 256, 2047]]))
    _check(c, out, rows=rows)


def test_zero_adapter_and_zero_weight():
    """B = 0 leaves the base output and gives dA = 0; W = 0 isolates the adapter."""
    c = Case(256, 256, 40, 8, seed=3)
    c.Bb = np.zeros_like(c.Bb)
    c.B = nf4.bf16_bits_to_f32(c.Bb)
    out = c.gpu()
    _check(c, out)
    assert torch.count_nonzero(out["dA"]).item() == 0
    c2 = Case(256, 256, 40, 8, seed=4)
    c2.W = np.zeros_like(c2.W)
    _check(c2, c2.gpu())


def test_deterministic():
    c = Case(776, 640, 300, 64, seed=5)
    a, b = c.gpu(), c.gpu()
    for k in ("Y", "XA", "dX", "dA", "dB"):
        assert torch.equal(a[k], b[k]), k


def test_no_tokens_backward_zeroes_adapter_grads():
    q = _q()
    K, N, r = 128, 64, 8
    dA = torch.full((K, r), 3.0, dtype=torch.bfloat16, device="cuda")
    dB = torch.full((r, N), 3.0, dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros(N * K // 2, dtype=torch.uint8, device="cuda")
    q8 = torch.zeros(N * K // 64, dtype=torch.uint8, device="cuda")
    s2 = torch.zeros((N * K // 64 + 255) // 256, dtype=torch.float32, device="cuda")
    X = torch.empty(0, K, dtype=torch.bfloat16, device="cuda")
    dY = torch.empty(0, N, dtype=torch.bfloat16, device="cuda")
    XA = torch.empty(0, r, dtype=torch.float32, device="cuda")
    A = torch.zeros(K, r, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(r, N, dtype=torch.bfloat16, device="cuda")
    q.linear_bwd(dY, X, XA, codes, q8, s2, A, B, 16.0, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dA).item() == 0 and torch.count_nonzero(dB).item() == 0


def test_argument_errors_raise():
    q = _q()
    X = torch.zeros(4, 96, dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros(64 * 96 // 2, dtype=torch.uint8, device="cuda")
    q8 = torch.zeros(96, dtype=torch.uint8, device="cuda")
    s2 = torch.zeros(1, dtype=torch.float32, device="cuda")
    A = torch.zeros(96, 8, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(q.QLoRAError):
        q.linear_fwd(X, codes, q8, s2, A, B, 16.0, 64)   # K = 96 is not a multiple of 64


def _random_single_cases(n, seed=4242):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        N = int(rng.integers(1, 300)) * 8
        K = int(rng.integers(1, 36)) * 64
        # half the cases on the small-token path (T <= 16), half above it
        T = int(rng.integers(1, 17)) if i % 2 == 0 else int(rng.integers(17, 600))
        r = int(rng.choice([8, 16, 24, 40, 64, 72, 96, 128]))
        cases.append((N, K, T, r))
    return cases


@pytest.mark.parametrize("N,K,T,r", _random_single_cases(8))
def test_random_shapes_against_oracle(N, K, T, r):
    """Seeded random single linears (N up to ~2400, K up to ~2200, T on both
    sides of the small-token boundary, ranks 8-128): codes and constants bit
    for bit, Y, XA, dX on sampled rows and dA, dB in full against the
    oracle."""
    print(f"random single N={N} K={K} T={T} r={r}", flush=True)
    c = Case(N, K, T, r, seed=N * 3 + K + T)
    rows = np.unique(np.array([0, T // 3, T // 2, T - 1]))
    _check(c, c.gpu(), rows=rows)
