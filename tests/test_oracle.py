"""Pins for the CPU oracle, checked against things other than itself.

Each test pins the oracle to an independent fact: hand-derived golden values,
an exact rational brute force, closed forms, invariants of the definition, or
a library routine (torch's rounding) for a special case. None of them needs a
GPU or the HIP library.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import gemm_oracle as go
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ helpers -------

def _bits_from_values(vals, dtype_code):
    t = torch.tensor(np.asarray(vals, dtype=np.float32))
    t = t.half() if dtype_code == 0 else t.bfloat16()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _exact_value(bits16, dtype_code):
    """Exact rational value of a 16-bit float pattern, from the bit fields."""
    b = int(bits16)
    if dtype_code == 0:
        sign, exp, man = b >> 15, (b >> 10) & 0x1F, b & 0x3FF
        assert exp != 0x1F
        v = Fraction(man, 1024) * Fraction(2) ** -14 if exp == 0 else \
            (1 + Fraction(man, 1024)) * Fraction(2) ** (exp - 15)
    else:
        sign, exp, man = b >> 15, (b >> 7) & 0xFF, b & 0x7F
        assert exp != 0xFF
        v = Fraction(man, 128) * Fraction(2) ** -126 if exp == 0 else \
            (1 + Fraction(man, 128)) * Fraction(2) ** (exp - 127)
    return -v if sign else v


def _brute_force(M, N, K, dt, tA, tB, alpha, beta, A, lda, B, ldb, C, ldc):
    """Exact D by a triple loop over Fractions, indexing the stored buffers directly."""
    D = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                a = A[k * lda + i] if tA else A[i * lda + k]
                b = B[j * ldb + k] if tB else B[k * ldb + j]
                s += _exact_value(a, dt) * _exact_value(b, dt)
            d = Fraction(alpha) * s
            if beta != 0:
                d += Fraction(beta) * Fraction(float(C[i * ldc + j]))
            D[i][j] = d
    return D


def _rand_case(rng, M, N, K, dt, tA, tB, pad=3):
    lda = (M if tA else K) + pad
    ldb = (K if tB else N) + pad
    ldc = N + pad
    a_rows = K if tA else M
    b_rows = N if tB else K
    A = _bits_from_values(rng.uniform(-1, 1, a_rows * lda), dt)
    B = _bits_from_values(rng.uniform(-1, 1, b_rows * ldb), dt)
    C = rng.uniform(-1, 1, M * ldc).astype(np.float32)
    return A, lda, B, ldb, C, ldc


# ------------------------------------------------------------ rounding ------

def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split()[:2])
    return rows


def _parse_value(s):
    # values such as "1+3*p-11" mean 1 + 3*2^-11, written exactly
    expr = s.replace("p-", "2.0**-")
    return float(eval(expr, {"__builtins__": {}}))  # fixture text is ours


def test_bf16_rounding_matches_hand_table():
    rows = _read_table("bf16_rounding.txt")
    assert len(rows) >= 15
    src = np.array([int(a, 16) for a, _ in rows], dtype=np.uint32).view(np.float32)
    want = np.array([int(b, 16) for _, b in rows], dtype=np.uint16)
    got = oracle.round_f32_to_bf16_bits(src)
    assert np.array_equal(got, want), [(hex(a), hex(b)) for a, b in zip(got, want) if a != b]


def test_f16_rounding_matches_hand_table():
    rows = _read_table("f16_rounding.txt")
    assert len(rows) >= 10
    src = np.array([_parse_value(a) for a, _ in rows], dtype=np.float32)
    want = np.array([int(b, 16) for _, b in rows], dtype=np.uint16)
    got = oracle.round_f32_to_f16_bits(src)
    assert np.array_equal(got, want)


def test_bf16_rounding_keeps_nan_nan():
    src = np.array([0x7FC00000, 0x7F800001, 0xFFC00001], dtype=np.uint32).view(np.float32)
    got = oracle.round_f32_to_bf16_bits(src)
    assert np.all(np.isnan(oracle.decode_bits(got, oracle.BF16)))


@pytest.mark.parametrize("dt", [0, 1])
def test_rounding_bitwise_equals_torch(dt):
    """Special case that reduces to a library routine: torch's f32->f16/bf16 cast."""
    rng = np.random.default_rng(5)
    parts = [
        rng.uniform(-1, 1, 200000).astype(np.float32),
        rng.standard_normal(100000).astype(np.float32) * 1e3,
        rng.standard_normal(100000).astype(np.float32) * 1e-6,
        # every 16-bit high half with assorted low halves, NaN excluded
        (np.arange(1 << 16, dtype=np.uint32)[:, None] << 16 |
         np.array([0, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)[None, :]).reshape(-1)
        .view(np.float32),
    ]
    x = np.concatenate(parts)
    x = x[~np.isnan(x)]
    want = _bits_from_values(x, dt)
    got = oracle.round_f32_bits(x, dt)
    assert np.array_equal(got, want)


def test_rounding_of_ragged_workload_source_equals_torch():
    cfg = workloads.CONFIGS["ragged4097x1000x1032_tn"]
    inp = workloads.make_inputs(workloads.with_shape(cfg, M=257, N=120, K=72))
    got = oracle.round_f32_bits(inp.A_src.numpy(), oracle.F16)
    assert np.array_equal(got, workloads.bits_u16(inp.A))


@pytest.mark.parametrize("dt", [0, 1])
def test_decode_every_pattern_matches_field_formula(dt):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.decode_bits(bits, dt)
    rng = np.random.default_rng(1)
    exp_all_ones = 0x7C00 if dt == 0 else 0x7F80
    for b in rng.choice(1 << 16, 3000, replace=False).tolist() + [0, 1, 0x8000, 0x3C00, 0x3F80]:
        if (b & exp_all_ones) == exp_all_ones:
            continue
        assert Fraction(float(vals[b])) == _exact_value(b, dt)


# ------------------------------------------------- brute force, exact -------

SHAPES = [(1, 1, 1), (2, 3, 1), (3, 2, 7), (7, 8, 15), (16, 8, 16), (8, 16, 17), (17, 3, 33),
          (15, 16, 2), (33, 2, 3)]


@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("dt", [0, 1])
def test_oracle_equals_exact_bruteforce(tA, tB, dt):
    rng = np.random.default_rng(100 + 10 * tA + 2 * tB + dt)
    for (M, N, K) in SHAPES:
        for alpha, beta in [(1.0, 0.0), (1.0, 1.0), (1.5, 0.5), (-2.0, -1.0)]:
            A, lda, B, ldb, C, ldc = _rand_case(rng, M, N, K, dt, tA, tB)
            D, bound = oracle.gemm_reference(M, N, K, dt, tA, tB, alpha, beta,
                                             A, lda, B, ldb, C, ldc)
            E = _brute_force(M, N, K, dt, tA, tB, alpha, beta, A, lda, B, ldb, C, ldc)
            for i in range(M):
                for j in range(N):
                    # fp64 summation of K+1 exact-ish terms: a few ulps of the bound
                    tol = (K + 3) * 2.0 ** -52 * bound[i, j]
                    assert abs(Fraction(D[i, j]) - E[i][j]) <= Fraction(tol), (M, N, K, i, j)


@pytest.mark.parametrize("tA,tB", [(0, 1), (1, 0)])
@pytest.mark.parametrize("dt", [0, 1])
def test_f32_operand_reference_equals_exact_on_library_rounding(tA, tB, dt):
    """float32 operands: the oracle's f32 entry (its own rounding, then the
    product) against exact Fraction sums of the values torch's rounding
    (`.half()` / `.bfloat16()`) gives each stored element. The sources are
    random float32 values, so almost every element actually rounds."""
    rng = np.random.default_rng(300 + 10 * tA + 2 * tB + dt)
    for (M, N, K) in [(3, 2, 7), (7, 8, 15), (8, 16, 17)]:
        for alpha, beta in [(1.0, 0.0), (-1.5, 0.5)]:
            lda, ldb, ldc = (M if tA else K) + 2, (K if tB else N) + 1, N
            Af = rng.uniform(-3, 3, (K if tA else M) * lda).astype(np.float32)
            Bf = rng.uniform(-3, 3, (N if tB else K) * ldb).astype(np.float32)
            C = rng.uniform(-1, 1, M * ldc).astype(np.float32)
            D, bound = oracle.gemm_reference_f32(M, N, K, dt, tA, tB, alpha, beta,
                                                 Af, lda, Bf, ldb, C, ldc)
            tdt = torch.float16 if dt == 0 else torch.bfloat16
            A16 = torch.tensor(Af).to(tdt).view(torch.int16).numpy().view(np.uint16)
            B16 = torch.tensor(Bf).to(tdt).view(torch.int16).numpy().view(np.uint16)
            assert np.mean(A16 != oracle.round_f32_bits(Af * 0 + 1, dt)) > 0.5  # not all ones
            E = _brute_force(M, N, K, dt, tA, tB, alpha, beta, A16, lda, B16, ldb, C, ldc)
            for i in range(M):
                for j in range(N):
                    tol = (K + 3) * 2.0 ** -52 * bound[i, j]
                    assert abs(Fraction(D[i, j]) - E[i][j]) <= Fraction(tol), (M, N, K, i, j)


# -------------------------------------------------------- 8-bit floats ----

def _fp8_value(text):
    if text in ("nan", "inf", "-inf", "-0"):
        return float(text)
    if "*p" in text:
        a, b = text.split("*p")
        return float(a) * 2.0 ** int(b)
    return float(text)


def test_fp8_decode_matches_hand_table():
    n = 0
    with open(os.path.join(GOLDEN, "fp8_codes.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if not line:
                continue
            fmt, code, val = line[0], int(line[1], 16), _fp8_value(line[2])
            got = oracle.decode_fp8(np.array([code]), 4 if fmt == "e4m3" else 5)[0]
            if np.isnan(val):
                assert np.isnan(got), (fmt, hex(code))
            else:
                assert got == val and np.signbit(got) == np.signbit(val), (fmt, hex(code), got)
            n += 1
    assert n >= 20


@pytest.mark.parametrize("dt,tdt", [(4, "float8_e4m3fn"), (5, "float8_e5m2")])
def test_fp8_decode_every_code_equals_torch(dt, tdt):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_fp8(codes, dt)
    lib = torch.from_numpy(codes).view(getattr(torch, tdt)).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], lib[ok])


@pytest.mark.parametrize("dt,tdt", [(4, "float8_e4m3fn"), (5, "float8_e5m2")])
@pytest.mark.parametrize("tA,tB", [(0, 1), (1, 0)])
def test_fp8_reference_equals_exact_on_library_values(dt, tdt, tA, tB):
    """The product on 8-bit float codes against exact Fraction sums of the
    values torch decodes them to."""
    rng = np.random.default_rng(700 + dt + 2 * tA)
    finite = [c for c in range(256) if np.isfinite(oracle.decode_fp8(np.array([c]), dt)[0])]
    for (M, N, K) in [(3, 2, 7), (8, 5, 33)]:
        lda, ldb, ldc = (M if tA else K) + 1, (K if tB else N) + 2, N
        A = rng.choice(finite, (K if tA else M) * lda).astype(np.uint8)
        B = rng.choice(finite, (N if tB else K) * ldb).astype(np.uint8)
        C = rng.uniform(-1, 1, M * ldc).astype(np.float32)
        D, bound = oracle.gemm_reference(M, N, K, dt, tA, tB, 0.5, -1.0, A, lda, B, ldb, C, ldc)
        av = torch.from_numpy(A).view(getattr(torch, tdt)).double().numpy()
        bv = torch.from_numpy(B).view(getattr(torch, tdt)).double().numpy()
        for i in range(M):
            for j in range(N):
                s = Fraction(0)
                for k in range(K):
                    a = av[k * lda + i] if tA else av[i * lda + k]
                    b = bv[j * ldb + k] if tB else bv[k * ldb + j]
                    s += Fraction(float(a)) * Fraction(float(b))
                e = Fraction(0.5) * s + Fraction(-1.0) * Fraction(float(C[i * ldc + j]))
                tol = (K + 3) * 2.0 ** -52 * bound[i, j]
                assert abs(Fraction(D[i, j]) - e) <= Fraction(tol), (M, N, K, i, j)


# ------------------------------------------------------- int8 -> int32 ----

def _wrap32(v: int) -> int:
    v &= 0xFFFFFFFF
    return v - (1 << 32) if v >= (1 << 31) else v


def _brute_force_i8(M, N, K, tA, tB, alpha, beta, A, lda, B, ldb, C, ldc):
    """Python-integer triple loop over the stored int8 buffers, then int32 wrap."""
    D = np.zeros((M, N), dtype=np.int64)
    for i in range(M):
        for j in range(N):
            s = 0
            for k in range(K):
                a = int(A[k * lda + i] if tA else A[i * lda + k])
                b = int(B[j * ldb + k] if tB else B[k * ldb + j])
                s += a * b
            d = alpha * s + (beta * int(C[i * ldc + j]) if beta != 0 else 0)
            D[i, j] = _wrap32(d)
    return D


@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_i8_oracle_equals_integer_bruteforce(tA, tB):
    rng = np.random.default_rng(500 + 2 * tA + tB)
    for (M, N, K) in [(1, 1, 1), (3, 2, 7), (7, 8, 33), (16, 5, 64)]:
        for alpha, beta in [(1, 0), (1, 1), (-3, 2), (2**31 - 1, -2**31), (7, -1)]:
            lda, ldb, ldc = (M if tA else K) + 2, (K if tB else N) + 3, N + 1
            A = rng.integers(-128, 128, (K if tA else M) * lda).astype(np.int8)
            B = rng.integers(-128, 128, (N if tB else K) * ldb).astype(np.int8)
            C = rng.integers(-2**31, 2**31, M * ldc).astype(np.int32)
            D = oracle.gemm_reference_i8(M, N, K, tA, tB, alpha, beta, A, lda, B, ldb, C, ldc)
            E = _brute_force_i8(M, N, K, tA, tB, alpha, beta, A, lda, B, ldb, C, ldc)
            assert D.dtype == np.int32 and np.array_equal(D.astype(np.int64), E), (M, N, K, alpha)


def test_i8_oracle_wraps_like_int32_and_skips_c():
    # 127*127*K exceeds 2^31 for K = 140000: the int32 sum wraps
    M, N, K = 2, 3, 140000
    A = np.full(M * K, 127, np.int8)
    B = np.full(N * K, 127, np.int8)
    D = oracle.gemm_reference_i8(M, N, K, 0, 1, 1, 0, A, K, B, K)
    assert np.all(D == _wrap32(127 * 127 * K)) and _wrap32(127 * 127 * K) < 0
    D = oracle.gemm_reference_i8(M, N, K, 0, 1, -1, 0, A, K, B, K)
    assert np.all(D == _wrap32(-127 * 127 * K))
    A = np.full(M * K, -128, np.int8)
    D = oracle.gemm_reference_i8(M, N, K, 0, 1, 1, 0, A, K, B, K)
    assert np.all(D == _wrap32(-128 * 127 * K))
    # beta == 0 never reads C; K == 0 and alpha == 0 give beta*C
    D = oracle.gemm_reference_i8(M, N, 5, 0, 0, 1, 0, A[:10], 5, B[:15], 3, None, None)
    assert np.all(D == 5 * (-128) * 127)
    C = np.arange(M * N, dtype=np.int32) - 3
    for K0, al in [(0, 1), (4, 0)]:
        D = oracle.gemm_reference_i8(M, N, K0, 0, 0, al, 3, A[:8], 4, B[:12], 3, C, N)
        assert np.array_equal(D.reshape(-1), 3 * C)


def test_i8_oracle_transpose_equivalence_and_ones():
    rng = np.random.default_rng(9)
    M, N, K = 9, 11, 40
    a = rng.integers(-128, 128, (M, K)).astype(np.int8)
    b = rng.integers(-128, 128, (K, N)).astype(np.int8)
    ref = oracle.gemm_reference_i8(M, N, K, 0, 0, 1, 0, a.reshape(-1), K, b.reshape(-1), N)
    assert np.array_equal(ref, oracle.gemm_reference_i8(
        M, N, K, 1, 1, 1, 0, a.T.copy().reshape(-1), M, b.T.copy().reshape(-1), K))
    assert np.array_equal(ref.astype(np.int64), a.astype(np.int64) @ b.astype(np.int64))
    ones = oracle.gemm_reference_i8(4, 5, 300, 0, 1, 1, 0, np.ones(1200, np.int8), 300,
                                    np.ones(1500, np.int8), 300)
    assert np.all(ones == 300)


def test_single_atom_16x8x16_workload_exact():
    cfg = workloads.CONFIGS["atom16x8x16"]
    inp = workloads.make_inputs(cfg)
    A, B = workloads.bits_u16(inp.A).reshape(-1), workloads.bits_u16(inp.B).reshape(-1)
    D, bound = oracle.gemm_reference(16, 8, 16, 0, 0, 0, 1.0, 0.0, A, 16, B, 8)
    E = _brute_force(16, 8, 16, 0, 0, 0, 1.0, 0.0, A, 16, B, 8, None, 8)
    for i in range(16):
        for j in range(8):
            assert abs(Fraction(D[i, j]) - E[i][j]) <= Fraction(19 * 2.0 ** -52 * bound[i, j])


def test_worked_example_fixture():
    vals = {}
    with open(os.path.join(GOLDEN, "worked_2x3x2.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                vals[line[0]] = [float(v) for v in line[1:]]
    M, N, K = int(vals["M"][0]), int(vals["N"][0]), int(vals["K"][0])
    for dt in (0, 1):
        A = _bits_from_values(vals["A"], dt)
        B = _bits_from_values(vals["B"], dt)
        C = np.array(vals["C"], dtype=np.float32)
        D, _ = oracle.gemm_reference(M, N, K, dt, 0, 0, vals["alpha"][0], vals["beta"][0],
                                     A, K, B, N, C, N)
        assert np.array_equal(D.reshape(-1), np.array(vals["D"]))
        # the same product with both operands stored transposed
        At = _bits_from_values(np.array(vals["A"]).reshape(M, K).T.reshape(-1), dt)
        Bt = _bits_from_values(np.array(vals["B"]).reshape(K, N).T.reshape(-1), dt)
        D2, _ = oracle.gemm_reference(M, N, K, dt, 1, 1, vals["alpha"][0], vals["beta"][0],
                                      At, M, Bt, K, C, N)
        assert np.array_equal(D2.reshape(-1), np.array(vals["D"]))


# ------------------------------------------------ closed forms, invariants ---

@pytest.mark.parametrize("dt", [0, 1])
def test_identity_and_permutation_are_exact(dt):
    rng = np.random.default_rng(7)
    M, K, N = 37, 29, 23
    A = _bits_from_values(rng.uniform(-1, 1, M * K), dt)
    Avals = oracle.decode_bits(A, dt).reshape(M, K)
    I = _bits_from_values(np.eye(K).reshape(-1), dt)
    D, _ = oracle.gemm_reference(M, K, K, dt, 0, 0, 1.0, 0.0, A, K, I, K)
    assert np.array_equal(D, Avals)
    # row permutation on the left, column permutation on the right
    p = rng.permutation(M)
    P = np.zeros((M, M))
    P[np.arange(M), p] = 1
    Pb = _bits_from_values(P.reshape(-1), dt)
    D, _ = oracle.gemm_reference(M, K, M, dt, 0, 0, 1.0, 0.0, Pb, M, A, K)
    assert np.array_equal(D, Avals[p, :])
    q = rng.permutation(K)
    Q = np.zeros((K, K))
    Q[q, np.arange(K)] = 1
    Qb = _bits_from_values(Q.reshape(-1), dt)
    D, _ = oracle.gemm_reference(M, K, K, dt, 0, 0, 1.0, 0.0, A, K, Qb, K)
    assert np.array_equal(D, Avals[:, q])


def test_ones_closed_form():
    M, N, K = 9, 11, 300
    A = _bits_from_values(np.ones(M * K), 1)
    B = _bits_from_values(np.ones(K * N), 1)
    C = np.full(M * N, 0.25, dtype=np.float32)
    D, bound = oracle.gemm_reference(M, N, K, 1, 0, 0, -2.0, 4.0, A, K, B, N, C, N)
    assert np.all(D == -2.0 * K + 1.0)
    assert np.all(bound == 2.0 * K + 1.0)


def test_integer_products_exact():
    """Integer operands: every partial sum is an exactly representable integer."""
    rng = np.random.default_rng(3)
    M, N, K = 20, 30, 500
    a = rng.integers(-2, 3, (M, K))
    b = rng.integers(-2, 3, (K, N))
    D, _ = oracle.gemm_reference(M, N, K, 0, 0, 0, 1.0, 0.0,
                                 _bits_from_values(a.reshape(-1), 0), K,
                                 _bits_from_values(b.reshape(-1), 0), N)
    want = np.zeros((M, N), dtype=np.int64)
    for k in range(K):  # integer arithmetic, no floating point at all
        want += np.outer(a[:, k], b[k, :])
    assert np.array_equal(D, want.astype(np.float64))


def test_beta_one_is_product_plus_c_and_alpha_scales():
    rng = np.random.default_rng(11)
    M, N, K = 31, 17, 45
    A, lda, B, ldb, C, ldc = _rand_case(rng, M, N, K, 1, 0, 1)
    D1, _ = oracle.gemm_reference(M, N, K, 1, 0, 1, 1.0, 1.0, A, lda, B, ldb, C, ldc)
    D0, _ = oracle.gemm_reference(M, N, K, 1, 0, 1, 1.0, 0.0, A, lda, B, ldb, C, ldc)
    Cm = C.reshape(M, ldc)[:, :N].astype(np.float64)
    assert np.array_equal(D1, D0 + Cm)
    D2, _ = oracle.gemm_reference(M, N, K, 1, 0, 1, 2.0, 0.0, A, lda, B, ldb, C, ldc)
    assert np.array_equal(D2, 2.0 * D0)


def test_beta_zero_does_not_read_c():
    rng = np.random.default_rng(12)
    M, N, K = 5, 6, 7
    A, lda, B, ldb, C, ldc = _rand_case(rng, M, N, K, 0, 0, 0)
    Cnan = np.full_like(C, np.nan)
    D, bound = oracle.gemm_reference(M, N, K, 0, 0, 0, 1.0, 0.0, A, lda, B, ldb, Cnan, ldc)
    assert np.all(np.isfinite(D)) and np.all(np.isfinite(bound))
    D, _ = oracle.gemm_reference(M, N, K, 0, 0, 0, 1.0, 0.0, A, lda, B, ldb, None, None)
    assert np.all(np.isfinite(D))


def test_k_zero_and_alpha_zero_give_beta_c():
    rng = np.random.default_rng(13)
    M, N = 4, 9
    C = rng.uniform(-1, 1, M * N).astype(np.float32)
    Cm = C.reshape(M, N).astype(np.float64)
    D, _ = oracle.gemm_reference(M, N, 0, 0, 0, 0, 1.0, -0.5, None, 1, None, 1, C, N)
    assert np.array_equal(D, -0.5 * Cm)
    A = _bits_from_values(np.full(M * 3, np.inf), 0)  # never read when alpha == 0
    D, _ = oracle.gemm_reference(M, N, 3, 0, 0, 0, 0.0, 2.0, A, 3, A, N, C, N)
    assert np.array_equal(D, 2.0 * Cm)


@pytest.mark.parametrize("dt", [0, 1])
def test_transpose_equivalence_exact(dt):
    rng = np.random.default_rng(21 + dt)
    M, N, K = 13, 19, 40
    a = rng.uniform(-1, 1, (M, K))
    b = rng.uniform(-1, 1, (K, N))
    C = rng.uniform(-1, 1, M * N).astype(np.float32)
    ref, _ = oracle.gemm_reference(M, N, K, dt, 0, 0, 1.5, -1.0,
                                   _bits_from_values(a.reshape(-1), dt), K,
                                   _bits_from_values(b.reshape(-1), dt), N, C, N)
    for tA in (0, 1):
        for tB in (0, 1):
            As = a.T if tA else a
            Bs = b.T if tB else b
            D, _ = oracle.gemm_reference(M, N, K, dt, tA, tB, 1.5, -1.0,
                                         _bits_from_values(As.reshape(-1), dt), As.shape[1],
                                         _bits_from_values(Bs.reshape(-1), dt), Bs.shape[1],
                                         C, N)
            assert np.array_equal(D, ref)


def test_rows_and_elements_agree_with_full():
    rng = np.random.default_rng(31)
    M, N, K = 70, 50, 64
    A, lda, B, ldb, C, ldc = _rand_case(rng, M, N, K, 1, 1, 0)
    full, fb = oracle.gemm_reference(M, N, K, 1, 1, 0, 2.0, -1.0, A, lda, B, ldb, C, ldc, slab=16)
    rows = np.array([0, 5, 69, 33])
    part, pb = oracle.gemm_reference(M, N, K, 1, 1, 0, 2.0, -1.0, A, lda, B, ldb, C, ldc,
                                     rows=rows)
    assert np.array_equal(part, full[rows]) and np.array_equal(pb, fb[rows])
    I = rng.integers(0, M, 40)
    J = rng.integers(0, N, 40)
    e, eb = oracle.gemm_reference_elements(M, N, K, 1, 1, 0, 2.0, -1.0, A, lda, B, ldb,
                                           C, ldc, I, J)
    assert np.allclose(e, full[I, J], rtol=0, atol=1e-13)
    assert np.allclose(eb, fb[I, J], rtol=0, atol=1e-13)


def test_check_tolerance_edges():
    ref = np.array([1.0, -2.0, 0.0])
    bound = np.array([10.0, 4.0, 0.0])
    tol = 2e-3 * bound + 1e-6
    assert oracle.check(ref + 0.99 * tol, ref, bound)["ok"]
    r = oracle.check(ref + np.array([0, 1.01 * tol[1], 0]), ref, bound)
    assert not r["ok"] and r["n_fail"] == 1 and r["first_fail"] == 1
    assert not oracle.check(np.array([1.0, np.nan, 0.0]), ref, bound)["ok"]


# --------------------------------- planted mistakes are caught by the pins ---

@pytest.mark.parametrize("mutant", ["transposed_a", "dropped_k", "beta_sign", "c_read_at_beta0"])
def test_pins_catch_planted_oracle_mistakes(monkeypatch, mutant):
    """Plant a plausible mistake in the oracle (CPU only) and require a pin to fail."""
    rng = np.random.default_rng(41)
    M, N, K = 7, 5, 9
    dt, tA, tB = 0, 1, 0
    A, lda, B, ldb, C, ldc = _rand_case(rng, M, N, K, dt, tA, tB)
    alpha, beta = 1.5, 0.5 if mutant != "c_read_at_beta0" else 0.0
    orig_op_a = go.op_a
    if mutant == "transposed_a":
        monkeypatch.setattr(go, "op_a", lambda *a: orig_op_a(*a)[::-1])
    elif mutant == "dropped_k":
        def bad(*a):
            x = orig_op_a(*a).copy()
            x[:, -1] = 0
            return x
        monkeypatch.setattr(go, "op_a", bad)
    elif mutant == "beta_sign":
        orig_c = go.c_matrix
        monkeypatch.setattr(go, "c_matrix", lambda *a: -orig_c(*a))
    elif mutant == "c_read_at_beta0":
        orig_ref = go.gemm_reference

        def bad_ref(*args, **kw):
            D, b = orig_ref(*args, **kw)
            Cm = go.c_matrix(args[12], args[0], args[1], args[13])
            return D + Cm, b
        monkeypatch.setattr(go, "gemm_reference", bad_ref)
    D, bound = go.gemm_reference(M, N, K, dt, tA, tB, alpha, beta, A, lda, B, ldb, C, ldc)
    E = _brute_force(M, N, K, dt, tA, tB, alpha, beta, A, lda, B, ldb, C, ldc)
    worst = max(abs(Fraction(D[i, j]) - E[i][j]) for i in range(M) for j in range(N))
    assert worst > Fraction(1, 1 << 20), "planted mistake went unnoticed"
