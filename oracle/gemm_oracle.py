"""CPU oracle for the dense contraction D = alpha*op(A)@op(B) + beta*C.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or load
this module: only the tests, the package's smoke check and the benchmark's
CPU-baseline leg use it. It shares no code, tables or constants with the HIP
library; the two meet only through the seeded inputs the tests hand to both.

What it computes, and where each step comes from:

* The contraction itself is the plain definition of the TIRx ``gemm`` tile
  primitive (Apache TVM docs, TIRx tile primitives, ``gemm``: opening
  paragraph), with the general scalars of the Phobos ``gemm`` example kernel
  (Phobos docs, ``@tensorcore``: the sm_75/sm_80 kernel pair, whose epilogue
  stores ``alpha * acc + beta * c_old``).
* The transpose flags only describe the stored orientation; A is normalised to
  [M,K] and B to [K,N] (TVM ``gemm`` page, "Algorithm" step 1, and its Chinese
  restatement, section 2, "dimension consistency").
* beta == 0 means C is not read: D starts from zero instead of from C (TVM
  ``gemm`` page, "How inputs change the algorithm", beta row, and "Algorithm"
  step 3).
* Operands are f16 or bf16 values and the accumulator is f32 on the device
  (TVM ``gemm`` page, "What it accepts", dtype row); the oracle instead forms
  every sum exactly enough in float64, so that the device result can be judged
  against it with an error bound.
* Operands that start as float32 are rounded to f16/bf16 first (Phobos
  ``@tensorcore``: "The forms", the sentence on rounding operands to f16);
  round-to-nearest-even is the reading taken, as the page names no mode.

* 8-bit float operands (dtypes 4 and 5, ``decode_fp8``): the fp8 precisions
  the ``gemm_async`` variants list (TVM ``gemm`` page, restated, the
  precision list); the operands are stored codes, decoded exactly, and the
  product is the same definition.
* int8 operands with an int32 result (``gemm_reference_i8``): the integer
  tensor-core form of the same contraction (Phobos ``@tensorcore``: "When it
  declines", the note on i8); sums taken exactly in int64 and wrapped to
  int32, the reading taken for an overflow rule the pages do not state.

Every step uses numpy in float64 (int64 for int8); the only library primitive
is ``np.matmul``.
There is no blocking beyond splitting rows into slabs to bound memory, which
does not change any individual dot product.
"""
from __future__ import annotations

import numpy as np

F16 = 0
BF16 = 1
F8E4M3 = 4  # 8-bit float operands (OCP E4M3), f32 accumulator and C/D
F8E5M2 = 5  # 8-bit float operands (OCP E5M2)

# Per-element pass criterion for a device result (its own tolerance, written
# here rather than borrowed from the device side).
RTOL = 2e-3
ATOL = 1e-6


# ---------------------------------------------------------------- rounding --

def round_f32_to_f16_bits(x) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns, round-to-nearest-even.

    numpy's float32->float16 cast is the IEEE conversion (nearest-even, with
    subnormal results kept and overflow to infinity).
    """
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        return x.astype(np.float16).view(np.uint16)


def round_f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even.

    bfloat16 is the upper half of a binary32 word. Rounding to nearest-even on
    the dropped 16 bits is: add 0x7FFF plus the lowest kept bit, then shift.
    A carry out of the mantissa correctly bumps the exponent (and the largest
    finite values round to infinity). NaNs are kept NaN by forcing a quiet bit.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    is_nan = ((u & np.uint64(0x7F800000)) == np.uint64(0x7F800000)) & \
             ((u & np.uint64(0x007FFFFF)) != np.uint64(0))
    quiet = ((u >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def round_f32_bits(x, dtype: int) -> np.ndarray:
    if dtype == F16:
        return round_f32_to_f16_bits(x)
    if dtype == BF16:
        return round_f32_to_bf16_bits(x)
    raise ValueError(f"dtype code {dtype} is neither f16 (0) nor bf16 (1)")


def decode_fp8(codes, dtype: int) -> np.ndarray:
    """8-bit float codes -> their exact values as float64, from the field
    layout of the two OCP 8-bit formats:

    * E4M3 (dtype 4): sign, 4 exponent bits (bias 7), 3 mantissa bits;
      exponent 0 is subnormal (m * 2^-9); exponent 15 with mantissa 7 is NaN
      and there is no infinity (largest finite 448).
    * E5M2 (dtype 5): sign, 5 exponent bits (bias 15), 2 mantissa bits;
      exponent 0 is subnormal (m * 2^-16); exponent 31 is infinity (m = 0)
      or NaN.
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    if dtype == F8E4M3:
        e, m = (c >> 3) & 0xF, c & 0x7
        val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
        val = np.where((e == 15) & (m == 7), np.nan, val)
    elif dtype == F8E5M2:
        e, m = (c >> 2) & 0x1F, c & 0x3
        val = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.exp2(e - 15.0))
        val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    else:
        raise ValueError(f"dtype code {dtype} is not an 8-bit float (4 or 5)")
    return sign * val


def decode_bits(bits, dtype: int) -> np.ndarray:
    """16-bit patterns (8-bit codes for dtypes 4 and 5) -> exact float64 values."""
    if dtype in (F8E4M3, F8E5M2):
        return decode_fp8(bits, dtype)
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        with np.errstate(invalid="ignore"):
            return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"dtype code {dtype} is neither f16 (0) nor bf16 (1)")


# ------------------------------------------------------------- operand views --

def _stored_2d(flat: np.ndarray, rows: int, cols: int, ld: int) -> np.ndarray:
    """View a row-major buffer with leading dimension ``ld`` as [rows, cols].

    Element (r, c) is ``flat[r*ld + c]``. The buffer may end right after the
    last valid element of the last row.
    """
    flat = np.asarray(flat).reshape(-1)
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols), dtype=flat.dtype)
    need = (rows - 1) * ld + cols
    if flat.size < need:
        raise ValueError(f"buffer holds {flat.size} elements, needs {need}")
    if flat.size < rows * ld:
        flat = np.concatenate([flat, np.zeros(rows * ld - flat.size, dtype=flat.dtype)])
    return flat[: rows * ld].reshape(rows, ld)[:, :cols]


def op_a(A_bits, M: int, K: int, lda: int, transA: int, dtype: int) -> np.ndarray:
    """op(A) as float64 [M, K]: A[i*lda+k] when transA == 0, A[k*lda+i] when 1."""
    if transA:
        return decode_bits(_stored_2d(A_bits, K, M, lda), dtype).T
    return decode_bits(_stored_2d(A_bits, M, K, lda), dtype)


def op_b(B_bits, K: int, N: int, ldb: int, transB: int, dtype: int) -> np.ndarray:
    """op(B) as float64 [K, N]: B[k*ldb+j] when transB == 0, B[j*ldb+k] when 1."""
    if transB:
        return decode_bits(_stored_2d(B_bits, N, K, ldb), dtype).T
    return decode_bits(_stored_2d(B_bits, K, N, ldb), dtype)


def c_matrix(C, M: int, N: int, ldc: int) -> np.ndarray:
    return _stored_2d(np.asarray(C, dtype=np.float32), M, N, ldc).astype(np.float64)


# ------------------------------------------------------------------- oracle --

def gemm_reference(M, N, K, dtype, transA, transB, alpha, beta,
                   A_bits, lda, B_bits, ldb, C=None, ldc=None,
                   rows=None, slab: int = 512, with_bound: bool = True):
    """D_ref (and its error bound) in float64.

    ``rows`` optionally selects output rows (any index array); all N columns
    are produced for each selected row. Returns ``(D_ref, bound)`` with shape
    [len(rows), N] (or [M, N]); ``bound`` is None when ``with_bound`` is False.

    bound[i,j] = |alpha| * sum_k |a(i,k)|*|b(k,j)| + |beta*C[i,j]|, the scale
    against which a device result is judged.
    """
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.size
    D = np.zeros((R, N), dtype=np.float64)
    bound = np.zeros((R, N), dtype=np.float64) if with_bound else None
    if R == 0 or N == 0:
        return D, bound
    # alpha*acc: A and B are only read when they contribute.
    if K > 0 and alpha != 0.0:
        Bop = op_b(B_bits, K, N, ldb, transB, dtype)
        Babs = np.abs(Bop) if with_bound else None
        Aop_all = op_a(A_bits, M, K, lda, transA, dtype)
        for s in range(0, R, slab):
            r = rows[s:s + slab]
            Ar = Aop_all[r, :]
            D[s:s + slab] = float(alpha) * np.matmul(Ar, Bop)
            if with_bound:
                bound[s:s + slab] = abs(float(alpha)) * np.matmul(np.abs(Ar), Babs)
    # beta*C: C is not read at all when beta == 0.
    if beta != 0.0:
        Cm = c_matrix(C, M, N, ldc)[rows, :]
        D += float(beta) * Cm
        if with_bound:
            bound += np.abs(float(beta) * Cm)
    return D, bound


def gemm_reference_f32(M, N, K, dtype, transA, transB, alpha, beta,
                       A_f32, lda, B_f32, ldb, C=None, ldc=None, **kw):
    """D_ref and bound for float32 operands that are rounded to ``dtype``
    (f16 or bf16, round-to-nearest-even) before the product: the Phobos
    ``@tensorcore`` form where float32 tensors give up input precision to run
    on the tensor cores ("The forms"). Element (i, k) of a stored operand is
    rounded on its own, so rounding the whole stored buffer first is the same
    computation; then the product is the plain definition above."""
    A_bits = round_f32_bits(np.asarray(A_f32, dtype=np.float32).reshape(-1), dtype)
    B_bits = round_f32_bits(np.asarray(B_f32, dtype=np.float32).reshape(-1), dtype)
    return gemm_reference(M, N, K, dtype, transA, transB, alpha, beta, A_bits, lda, B_bits, ldb,
                          C, ldc, **kw)


def gemm_reference_i8(M, N, K, transA, transB, alpha, beta, A, lda, B, ldb, C=None, ldc=None,
                      rows=None):
    """int8 operands, int32 result: D = alpha*op(A)@op(B) + beta*C over the
    integers, reduced modulo 2^32 to two's-complement int32.

    The integer form of the same contraction: an i8 dot runs on the integer
    tensor cores whenever its shape allows (Phobos docs, ``@tensorcore``:
    "When it declines", the closing note on i8). The pages give no output
    type or overflow rule; the reading taken is an int32 accumulator whose
    sums, and the alpha/beta epilogue, wrap like int32 arithmetic. alpha and
    beta are integers; beta == 0 means C is not read; K == 0 or alpha == 0
    gives beta*C. ``A``/``B`` are the stored int8 buffers (flat, leading
    dimensions lda/ldb, same transpose formulas as the floating-point case).
    Returns the int32 [len(rows), N] result."""
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    mask = np.uint64(0xFFFFFFFF)
    acc = np.zeros((rows.size, N), dtype=np.uint64)
    if K > 0 and alpha != 0 and rows.size and N:
        a = _stored_2d(np.asarray(A, dtype=np.int8).reshape(-1), *((K, M) if transA else (M, K)), lda)
        b = _stored_2d(np.asarray(B, dtype=np.int8).reshape(-1), *((N, K) if transB else (K, N)), ldb)
        a = (a.T if transA else a).astype(np.int64)[rows, :]
        b = (b.T if transB else b).astype(np.int64)
        # |each sum| <= 2^14 * K < 2^45: exact in int64; then wrap to 32 bits
        prod = np.matmul(a, b).astype(np.uint64) & mask
        acc = (prod * (np.uint64(int(alpha) & 0xFFFFFFFF))) & mask
    if beta != 0 and rows.size and N:
        c = _stored_2d(np.asarray(C, dtype=np.int32).reshape(-1), M, N, ldc)[rows, :]
        acc = (acc + ((c.astype(np.int64).astype(np.uint64) & mask) *
                      np.uint64(int(beta) & 0xFFFFFFFF))) & mask
    return acc.astype(np.uint32).view(np.int32)


def gemm_reference_elements(M, N, K, dtype, transA, transB, alpha, beta,
                            A_bits, lda, B_bits, ldb, C, ldc, I, J):
    """D_ref and bound at individual (I[t], J[t]) positions, one dot product each."""
    I = np.asarray(I, dtype=np.int64)
    J = np.asarray(J, dtype=np.int64)
    D = np.zeros(I.size, dtype=np.float64)
    bound = np.zeros(I.size, dtype=np.float64)
    if K > 0 and alpha != 0.0:
        Aop = op_a(A_bits, M, K, lda, transA, dtype)
        Bop = op_b(B_bits, K, N, ldb, transB, dtype)
        for t in range(I.size):
            a = Aop[I[t], :]
            b = Bop[:, J[t]]
            D[t] = float(alpha) * float(np.dot(a, b))
            bound[t] = abs(float(alpha)) * float(np.dot(np.abs(a), np.abs(b)))
    if beta != 0.0:
        Cm = c_matrix(C, M, N, ldc)
        c = Cm[I, J]
        D += float(beta) * c
        bound += np.abs(float(beta) * c)
    return D, bound


def check(D, D_ref, bound, rtol: float = RTOL, atol: float = ATOL):
    """Elementwise |D - D_ref| <= rtol*bound + atol.

    Returns a dict with ``ok``, ``n_fail``, ``max_rel_err`` (max of
    |D-D_ref|/bound over elements with a nonzero bound), ``max_tol_ratio``
    (max of |D-D_ref|/(rtol*bound+atol); <= 1 passes) and the first failing
    flat index, if any.
    """
    D = np.asarray(D, dtype=np.float64)
    err = np.abs(D - D_ref)
    tol = rtol * bound + atol
    bad = ~(err <= tol)  # NaN counts as a failure
    nz = bound > 0
    max_rel = float(np.max(err[nz] / bound[nz])) if np.any(nz) else 0.0
    if np.any(~nz):
        max_rel = max(max_rel, float(np.max(np.where(err[~nz] > 0, np.inf, 0.0))))
    return {
        "ok": not bool(np.any(bad)),
        "n_fail": int(np.count_nonzero(bad)),
        "max_rel_err": max_rel,
        "max_tol_ratio": float(np.max(err / tol)) if err.size else 0.0,
        "first_fail": int(np.flatnonzero(bad)[0]) if np.any(bad) else None,
    }
