"""Pins of the CPU oracle against things other than itself.

Each test fixes one part of the oracle by a closed form, an invariant, an
exact brute-force sum, a published error bound or an independent library
routine, chosen so that a plausible slip (a dropped term, a swapped index, a
transposed operand, a wrong sign or rounding) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from dense_bf16_gemm_amd import synth

LAYOUTS = ["nn", "nt", "tn", "tt"]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_to_bits(x):
    """fp32 values that are exactly bf16-representable -> their bf16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def store(opA, opB, layout):
    """op(A) [M,K] and op(B) [K,N] (bf16 bits) -> storage arrays for ``layout``."""
    A = opA.T.copy() if layout in ("tn", "tt") else opA
    B = opB.T.copy() if layout in ("nt", "tt") else opB
    return np.ascontiguousarray(A), np.ascontiguousarray(B)


def rand_bits(shape, seed, sigma=1.0):
    return synth.bits(synth.randn_bf16(shape, sigma, seed))


def int_bits(shape, lo, hi, seed):
    return synth.bits(synth.randint_bf16(shape, lo, hi, seed))


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,K", [(1, 1), (7, 7), (64, 64), (129, 129), (5, 64)])
def test_identity_b_returns_a(layout, M, K):
    a = rand_bits((M, K), 11 + M)
    eye = f32_to_bits(np.eye(K, dtype=np.float32))
    A, B = store(a, eye, layout)
    y, bits = oracle.gemm(A, B, layout)
    np.testing.assert_array_equal(bits, a)
    np.testing.assert_array_equal(y, bits_to_f32(a))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_identity_a_returns_b(layout):
    b = rand_bits((33, 17), 5)
    eye = f32_to_bits(np.eye(33, dtype=np.float32))
    A, B = store(eye, b, layout)
    _, bits = oracle.gemm(A, B, layout)
    np.testing.assert_array_equal(bits, b)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 7, 7), (64, 64, 64), (129, 129, 129), (3, 5, 4096)])
def test_all_ones_gives_k(layout, M, N, K):
    one = np.uint16(0x3F80)
    A, B = store(np.full((M, K), one, np.uint16), np.full((K, N), one, np.uint16), layout)
    y, bits = oracle.gemm(A, B, layout)
    assert np.all(y == np.float32(K))
    want = torch.tensor(float(K)).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
    assert np.all(bits == want)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(7, 9, 64), (129, 17, 129), (16, 16, 1000)])
def test_rank_one_outer_product(layout, M, N, K):
    g = np.random.default_rng(M * 1000 + N + K)
    a = g.integers(-3, 4, M).astype(np.float32)
    b = g.integers(-3, 4, N).astype(np.float32)
    s = g.integers(-2, 3, K).astype(np.float32)
    t = g.integers(-2, 3, K).astype(np.float32)
    opA = f32_to_bits(np.outer(a, s))
    opB = f32_to_bits(np.outer(t, b))
    A, B = store(opA, opB, layout)
    y, _ = oracle.gemm(A, B, layout)
    want = np.outer(a, b) * float(np.dot(s, t))
    np.testing.assert_array_equal(y, want.astype(np.float32))


def test_golden_worked_examples():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        opA = f32_to_bits(np.array(c["A"], np.float32))
        opB = f32_to_bits(np.array(c["B"], np.float32))
        bias = f32_to_bits(np.array(c["bias"], np.float32)) if c.get("bias") is not None else None
        for layout in LAYOUTS:
            A, B = store(opA, opB, layout)
            y, _ = oracle.gemm(A, B, layout, c["epilogue"], bias=bias)
            np.testing.assert_array_equal(y, np.array(c["out"], np.float32), err_msg=c["name"])


# ------------------------------------------------------- exact brute force sums
@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny_integer_exact(seed):
    g = np.random.default_rng(seed)
    M, N, K = (int(v) for v in g.integers(1, 10, 3))
    opA = g.integers(-8, 9, (M, K)).astype(np.float32)
    opB = g.integers(-8, 9, (K, N)).astype(np.float32)
    for layout in LAYOUTS:
        A, B = store(f32_to_bits(opA), f32_to_bits(opB), layout)
        y, _ = oracle.gemm(A, B, layout)
        for i in range(M):
            for j in range(N):
                assert y[i, j] == math.fsum(opA[i, k] * opB[k, j] for k in range(K))


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_tiny_random_within_bound(seed):
    M, N, K = 5, 6, 9
    a = rand_bits((M, K), 100 + seed)
    b = rand_bits((K, N), 200 + seed)
    y, _ = oracle.gemm(a, b, "nn")
    af, bf = bits_to_f32(a).astype(np.float64), bits_to_f32(b).astype(np.float64)
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    for i in range(M):
        for j in range(N):
            exact = math.fsum(af[i, k] * bf[k, j] for k in range(K))
            absum = math.fsum(abs(af[i, k] * bf[k, j]) for k in range(K))
            assert abs(float(y[i, j]) - exact) <= gamma * absum


# ---------------------------------------------- recursive-summation error bound
@pytest.mark.parametrize("M,N,K", [(64, 64, 4096), (33, 17, 65536)])
def test_fp32_accumulation_within_higham_bound(M, N, K):
    """|y - y64| <= gamma_K * sum_k |a_ik b_kj| (recursive summation, u = 2^-24).

    Also rules out accumulating in bf16 or rounding partial sums: those exceed
    the bound by orders of magnitude at these K.
    """
    a = rand_bits((M, K), 7)
    bt = rand_bits((N, K), 8, sigma=K ** -0.5)
    y, _ = oracle.gemm(a, bt, "nt")
    af = bits_to_f32(a).astype(np.float64)
    bf = bits_to_f32(bt).astype(np.float64).T
    y64 = af @ bf
    absum = np.abs(af) @ np.abs(bf)
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    err = np.abs(y.astype(np.float64) - y64)
    assert np.all(err <= gamma * absum)
    # and the result is a genuine fp32 sum, not an exactly rounded one
    assert np.max(err) > 0


# ------------------------------------------------------------------ invariants
@pytest.mark.parametrize("M,N,K", [(257, 263, 1031)])
def test_rows_path_equals_literal_triple_loop(M, N, K):
    a = rand_bits((M, K), 31)
    b = rand_bits((K, N), 32, sigma=K ** -0.5)
    bias = rand_bits((N,), 33)
    for layout in LAYOUTS:
        A, B = store(a, b, layout)
        for epi in ("none", "bias_gelu_tanh"):
            y, bits = oracle.gemm(A, B, layout, epi, bias=bias)
            ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
            yp, bp = oracle.points(A, B, ii.ravel(), jj.ravel(), layout, epi, bias=bias)
            np.testing.assert_array_equal(yp.reshape(M, N), y)
            np.testing.assert_array_equal(bp.reshape(M, N), bits)


def test_rows_path_equals_literal_loop_wide():
    M, N, K = 64, 3001, 4096
    a = rand_bits((M, K), 41)
    bt = rand_bits((N, K), 42, sigma=K ** -0.5)
    y, _ = oracle.gemm(a, bt, "nt")
    rows, cols = synth.sample_points(M, N, 3000, 43)
    yp, _ = oracle.points(a, bt, rows, cols, "nt")
    np.testing.assert_array_equal(yp, y[rows, cols])


def test_row_range_matches_full():
    a = rand_bits((100, 70), 51)
    b = rand_bits((70, 90), 52)
    y, bits = oracle.gemm(a, b, "nn")
    y2, bits2 = oracle.gemm(a, b, "nn", rows=(37, 81))
    np.testing.assert_array_equal(y2, y[37:81])
    np.testing.assert_array_equal(bits2, bits[37:81])


def test_layouts_agree_bitwise():
    a = rand_bits((65, 300), 61)
    b = rand_bits((300, 47), 62)
    ref = None
    for layout in LAYOUTS:
        A, B = store(a, b, layout)
        y, _ = oracle.gemm(A, B, layout)
        if ref is None:
            ref = y
        np.testing.assert_array_equal(y, ref)


def test_layout_is_not_silently_transposed():
    """Square operands: op(B) must differ from storage when the layout says so."""
    a = rand_bits((16, 16), 71)
    b = rand_bits((16, 16), 72)
    y_nn, _ = oracle.gemm(a, b, "nn")
    y_nt, _ = oracle.gemm(a, b, "nt")  # uses b^T
    y_tn, _ = oracle.gemm(a, b, "tn")  # uses a^T
    af, bf = bits_to_f32(a).astype(np.float64), bits_to_f32(b).astype(np.float64)
    np.testing.assert_allclose(y_nn, af @ bf, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(y_nt, af @ bf.T, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(y_tn, af.T @ bf, rtol=1e-5, atol=1e-4)


# ------------------------------------------------------------------- epilogues
def test_bias_is_per_column_broadcast_over_rows():
    M = N = K = 24
    eye = f32_to_bits(np.eye(K, dtype=np.float32))
    b = int_bits((K, N), -50, 50, 81)
    bias = int_bits((N,), -60, 60, 82)
    y, _ = oracle.gemm(eye, b, "nn", "bias", bias=bias)
    want = bits_to_f32(b) + bits_to_f32(bias)[None, :]
    np.testing.assert_array_equal(y, want)


def test_gelu_tanh_matches_torch_float64():
    t = np.linspace(-12, 12, 200001, dtype=np.float32)
    y = oracle.gelu_tanh(t)
    ref = torch.nn.functional.gelu(torch.from_numpy(t).double(), approximate="tanh").float().numpy()
    ulp = np.spacing(np.abs(ref)).astype(np.float64)
    # below -7 the tanh form cancels (1 + tanh(z) with tanh(z) within 1e-16 of
    # -1): both evaluations are then only accurate to ~1e-16 absolute
    assert np.all(np.abs(y.astype(np.float64) - ref) <= ulp + 1e-14)
    assert np.all(y[t > -7] == ref[t > -7]) or np.all(np.abs(y - ref)[t > -7] <= ulp[t > -7])


def test_gelu_tanh_identities():
    t = np.linspace(-8, 8, 16001, dtype=np.float32)
    y = oracle.gelu_tanh(t).astype(np.float64)
    ym = oracle.gelu_tanh(-t).astype(np.float64)
    assert oracle.gelu_tanh(np.zeros(1, np.float32))[0] == 0.0
    # GELU(t) - GELU(-t) = t exactly in real arithmetic; fp32 rounding of each side only
    tol = 2 * np.spacing(np.maximum(np.abs(y), np.abs(ym)).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs((y - ym) - t.astype(np.float64)) <= tol + 1e-30)
    # tends to the identity / zero in the tails
    assert abs(oracle.gelu_tanh(np.array([20.0], np.float32))[0] - 20.0) == 0.0
    assert oracle.gelu_tanh(np.array([-20.0], np.float32))[0] <= 0.0


def test_silu_matches_torch_and_identity():
    g = np.linspace(-30, 30, 120001, dtype=np.float32)
    one = np.ones_like(g)
    y = oracle.silu_mul(g, one)
    ref = torch.nn.functional.silu(torch.from_numpy(g).double()).float().numpy()
    ulp = np.spacing(np.abs(ref)).astype(np.float64)
    assert np.all(np.abs(y.astype(np.float64) - ref) <= ulp)
    assert oracle.silu_mul(np.zeros(1, np.float32), np.ones(1, np.float32))[0] == 0.0
    s = np.linspace(-8, 8, 1601, dtype=np.float32)
    d = oracle.silu_mul(s, np.ones_like(s)).astype(np.float64) - oracle.silu_mul(-s, np.ones_like(s)).astype(np.float64)
    assert np.all(np.abs(d - s) <= 4 * np.spacing(np.abs(s)).astype(np.float64) + 1e-30)
    # the gate multiplies
    u = np.full_like(g, 3.0)
    np.testing.assert_allclose(oracle.silu_mul(g, u), 3.0 * ref, rtol=2e-7, atol=1e-30)


@pytest.mark.parametrize("epi", ["gelu_tanh", "bias_gelu_tanh"])
def test_gemm_epilogue_applies_activation_after_bias(epi):
    """Identity A: y[i][j] = act(B[i][j] (+ bias[j])), against torch float64."""
    K = N = 40
    eye = f32_to_bits(np.eye(K, dtype=np.float32))
    b = rand_bits((K, N), 91, sigma=2.0)
    bias = rand_bits((N,), 92)
    y, _ = oracle.gemm(eye, b, "nn", epi, bias=bias)
    t = bits_to_f32(b).astype(np.float32)
    if epi == "bias_gelu_tanh":
        t = (t + bits_to_f32(bias)[None, :]).astype(np.float32)  # fp32 add
    ref = torch.nn.functional.gelu(torch.from_numpy(t).double(), approximate="tanh").float().numpy()
    assert np.all(np.abs(y.astype(np.float64) - ref) <= np.spacing(np.abs(ref)))


def test_gemm_swiglu_gate_and_up_roles():
    """Identity x: y[i][j] = SiLU(Wg[j][i]) * Wu[j][i] (weights stored [N][K])."""
    K = M = 48
    N = 40
    eye = f32_to_bits(np.eye(K, dtype=np.float32))
    wg = rand_bits((N, K), 101, sigma=2.0)
    wu = rand_bits((N, K), 102, sigma=2.0)
    y, _ = oracle.gemm(eye, wg, "nt", "swiglu", B2=wu)
    g = torch.from_numpy(bits_to_f32(wg).T.copy()).double()
    u = torch.from_numpy(bits_to_f32(wu).T.copy()).double()
    ref = (torch.nn.functional.silu(g) * u).float().numpy()
    assert np.all(np.abs(y.astype(np.float64) - ref) <= np.spacing(np.abs(ref)))
    # swapping the roles changes the result (the gate is not symmetric)
    y_sw, _ = oracle.gemm(eye, wu, "nt", "swiglu", B2=wg)
    assert not np.array_equal(y, y_sw)
    yi, _ = oracle.gemm(eye, wg, "nt", "glu_identity", B2=wu)
    np.testing.assert_array_equal(yi, (bits_to_f32(wg).T * bits_to_f32(wu).T).astype(np.float32))


# ------------------------------------------------------------- bf16 rounding
def test_rne_tie_and_special_cases():
    cases = {
        0x3F808000: 0x3F80,  # tie, round down to even
        0x3F818000: 0x3F82,  # tie, round up to even
        0x3F808001: 0x3F81,  # above the tie
        0x3F807FFF: 0x3F80,  # below the tie
        0x7F7FFFFF: 0x7F80,  # max finite fp32 -> +inf
        0xFF7FFFFF: 0xFF80,
        0x7F800000: 0x7F80,  # inf stays inf
        0x00000000: 0x0000,
        0x80000000: 0x8000,
        0x00010000: 0x0001,  # smallest bf16 denormal
    }
    x = np.array(list(cases.keys()), np.uint32).view(np.float32)
    got = oracle.round_bf16(x)
    np.testing.assert_array_equal(got, np.array(list(cases.values()), np.uint16))
    nan = np.array([0x7FC00001, 0xFF800001, 0x7F800001], np.uint32).view(np.float32)
    r = oracle.round_bf16(nan)
    assert np.all((r & 0x7F80) == 0x7F80) and np.all((r & 0x007F) != 0)  # still NaN
    assert np.all((r & 0x0040) != 0)  # quiet
    assert (r[1] & 0x8000) != 0  # sign kept


def test_rne_matches_torch_on_structured_values():
    g = np.random.default_rng(123)
    hi = g.integers(0, 1 << 16, 2_000_000, dtype=np.uint32)
    lo = np.concatenate([
        np.full(400_000, 0x8000, np.uint32), np.full(400_000, 0x7FFF, np.uint32),
        np.full(400_000, 0x8001, np.uint32), g.integers(0, 1 << 16, 800_000, dtype=np.uint32),
    ])
    u = (hi << 16) | lo
    x = u.view(np.float32)
    finite = np.isfinite(x)
    x = x[finite]
    got = oracle.round_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_bf16_output_bits_are_rne_of_y():
    a = rand_bits((50, 300), 111)
    b = rand_bits((300, 60), 112)
    y, bits = oracle.gemm(a, b, "nn")
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


# ------------------------------------------------------------- argument errors
def test_rejects_mismatched_shapes():
    with pytest.raises(ValueError):
        oracle.gemm(rand_bits((4, 5), 1), rand_bits((6, 7), 2), "nn")
    with pytest.raises(RuntimeError):
        oracle.gemm(rand_bits((4, 5), 1), rand_bits((5, 7), 2), "nn", "bias")  # no bias


def test_empty_inputs():
    y, bits = oracle.gemm(np.zeros((0, 8), np.uint16), np.zeros((8, 5), np.uint16), "nn")
    assert y.shape == (0, 5)
    y, _ = oracle.gemm(np.zeros((3, 0), np.uint16), np.zeros((0, 5), np.uint16), "nn")
    assert np.all(y == 0)


def test_empty_sum_gives_the_epilogue_of_the_bias():
    """K = 0: each accumulator is the empty sum 0, so the bias epilogue
    returns the bias itself (its bf16 bits unchanged), GELU(bias) equals the
    oracle's GELU of those values, and the gated FFN gives act(0) * 0 = 0."""
    M, N = 5, 64
    bias = rand_bits((N,), 83)
    A, B = np.zeros((M, 0), np.uint16), np.zeros((N, 0), np.uint16)
    y, bits = oracle.gemm(A, B, "nt", "bias", bias=bias)
    np.testing.assert_array_equal(bits, np.broadcast_to(bias, (M, N)))
    np.testing.assert_array_equal(y, np.broadcast_to(bits_to_f32(bias), (M, N)))
    y, _ = oracle.gemm(A, B, "nt", "bias_gelu_tanh", bias=bias)
    np.testing.assert_array_equal(y, np.broadcast_to(oracle.gelu_tanh(bits_to_f32(bias)), (M, N)))
    for epi in ("none", "gelu_tanh"):
        y, bits = oracle.gemm(A, B, "nt", epi)
        assert np.all(y == 0) and np.all(bits == 0)
    for epi in ("swiglu", "glu_identity"):
        y, _ = oracle.gemm(A, B, "nt", epi, B2=B)
        assert np.all(y == 0)


# ---------------------------------------------------------------- non-finite inputs
def nonfinite_operands(M, N, K, seed):
    """op(A) [M,K], op(B) [K,N] bf16 bits: N(0,1)-like values with a few +-inf
    and NaN entries, and a zero of op(B) under an inf of op(A)."""
    a = bits_to_f32(rand_bits((M, K), seed)).copy()
    b = bits_to_f32(rand_bits((K, N), seed + 1)).copy()
    a[1, 2] = np.inf       # row 1: +-inf by the sign of b[2, j] ...
    b[2, 3] = 0.0          # ... and inf * 0 = NaN at (1, 3)
    a[2, 4] = np.nan       # row 2: NaN throughout
    b[5, 6] = -np.inf      # column 6: +-inf by the sign of a[i, 5]
    a[3, 7] = np.inf       # row 3: +inf and -inf terms where b[7, j] and
    a[3, 8] = -np.inf      # b[8, j] share a sign: NaN there
    return f32_to_bits(a), f32_to_bits(b)


def ieee_class(a, b):
    """Class of each entry of a @ b in any summation order: 0 finite, 1 +inf,
    -1 -inf, 2 NaN (terms NaN, inf * 0, or +inf and -inf together).  Finite
    terms are small, so no finite sum overflows."""
    with np.errstate(invalid="ignore", over="ignore"):
        t = a.astype(np.float64)[:, :, None] * b.astype(np.float64)[None, :, :]
    nan = np.isnan(t).any(1) | (np.isposinf(t).any(1) & np.isneginf(t).any(1))
    out = np.where(np.isposinf(t).any(1), 1, np.where(np.isneginf(t).any(1), -1, 0))
    return np.where(nan, 2, out)


def value_class(y):
    y = np.asarray(y, np.float64)
    return np.where(np.isnan(y), 2, np.where(np.isposinf(y), 1, np.where(np.isneginf(y), -1, 0)))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_nonfinite_inputs_follow_ieee(layout):
    """Inf and NaN inputs: every output's class (finite, +inf, -inf, NaN) is
    the one IEEE arithmetic fixes whatever the summation order, in the fp32
    result and in its bf16 bits; finite outputs match float64 within the
    fp32 accumulation bound."""
    M, N, K = 9, 11, 16
    ab, bb = nonfinite_operands(M, N, K, 21)
    a, b = bits_to_f32(ab), bits_to_f32(bb)
    A, B = store(ab, bb, layout)
    y, bits = oracle.gemm(A, B, layout)
    cls = ieee_class(a, b)
    assert {0, 1, -1, 2} <= set(np.unique(cls).tolist()), "the case should hold every class"
    np.testing.assert_array_equal(value_class(y), cls)
    np.testing.assert_array_equal(value_class(bits_to_f32(bits)), cls)
    fin = cls == 0
    with np.errstate(invalid="ignore"):
        ref = a.astype(np.float64) @ b.astype(np.float64)
        bound = 2 * K * np.finfo(np.float32).eps * (np.abs(a).astype(np.float64) @ np.abs(b)) + 1e-30
    assert np.all(np.abs(y[fin] - ref[fin]) <= bound[fin])


def test_nonfinite_through_the_epilogues():
    """GELU(+inf) = +inf, GELU(-inf) = NaN (the tanh form is -inf * 0 there),
    GELU(NaN) = NaN; SiLU(g) u and g u follow IEEE products."""
    t = np.array([np.inf, -np.inf, np.nan, 3.0], np.float32)
    g = oracle.gelu_tanh(t)
    assert g[0] == np.inf and np.isnan(g[1]) and np.isnan(g[2]) and np.isfinite(g[3])
    # through the full epilogue: a 1 x 4 output with K = 1, op(A) = [1], op(B) = t
    ones = f32_to_bits(np.ones((1, 1), np.float32))
    tb = f32_to_bits(t.reshape(1, 4))
    bias = f32_to_bits(np.zeros(4, np.float32))
    y, _ = oracle.gemm(ones, tb, "nn", "bias_gelu_tanh", bias=bias)
    assert y[0, 0] == np.inf and np.isnan(y[0, 1]) and np.isnan(y[0, 2])
    u = f32_to_bits(np.array([[2.0, 2.0, 2.0, 0.0]], np.float32))
    y, _ = oracle.gemm(ones, tb, "nn", "glu_identity", B2=u)
    assert y[0, 0] == np.inf and y[0, 1] == -np.inf and np.isnan(y[0, 2]) and y[0, 3] == 0.0
    y, _ = oracle.gemm(ones, tb, "nn", "swiglu", B2=u)
    # SiLU(+inf) = +inf, SiLU(-inf) = -inf / (1 + inf) = NaN
    assert y[0, 0] == np.inf and np.isnan(y[0, 1]) and np.isnan(y[0, 2])
