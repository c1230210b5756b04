"""Seeded random 8-bit calls against the oracle, across the planner's choices.

int8 (int32 C/D, bit-exact) and fp8 E4M3/E5M2 (f32 C/D, within the oracle's
bound): shapes, layouts, leading dimensions (16-byte rows or odd pitches),
an operand base one byte past a 16-byte boundary, alpha/beta and C == D are
drawn from a fixed seed, so every run checks the same calls. The planner
picks the kernel (two-group 256x256, whole or edge tiles, C/D by column
quads or element by element, or the 128x128 byte kernel with 16-byte or
bytewise staging); every result is compared over all of D, and the columns
past N must keep their sentinel.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import D_SENTINEL, need_gpu, say
from test_gemm_fp8_gpu import run_fp8
from test_gemm_i8_gpu import SENTINEL, run_i8

pytestmark = pytest.mark.gpu


def _draw(rng, size):
    if size == "small":
        M, N, K = (int(x) for x in rng.integers(1, [600, 600, 1100]))
    else:  # grids of 4 to 20 tiles of 256x256, K a multiple of 16 or not
        M, N = (int(x) for x in rng.integers(500, [1200, 1200]))
        if rng.random() < 0.6:  # M/N-contiguous operands in whole 16-byte pieces
            M, N = M // 16 * 16, N // 16 * 16
        K = int(rng.choice([128, 256, 384, 400, 520, 640]))
    tA, tB = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    pad = lambda x: (x + 15) // 16 * 16
    lda = M if tA else K
    ldb = K if tB else N
    aligned = 0.75 if size == "small" else 0.9
    lda = pad(lda) if rng.random() < aligned else lda + int(rng.integers(1, 4))
    ldb = pad(ldb) if rng.random() < aligned else ldb + int(rng.integers(1, 4))
    a_off = 1 if rng.random() < 0.1 else 0
    inplace = rng.random() < 0.25
    # rows of C/D 16-byte aligned (N a multiple of 4) or not
    ldd = N if inplace or rng.random() < 0.5 else N + int(rng.integers(1, 4))
    return M, N, K, tA, tB, lda, ldb, ldd, a_off, inplace


@pytest.mark.parametrize("size,block", [("small", 0), ("small", 1), ("mid", 0), ("mid", 1)])
def test_random_i8_calls(size, block, monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_PATH", raising=False)
    need_gpu()
    rng = np.random.default_rng(9090 + 10 * block + (size == "mid"))
    paths = set()
    for i in range(12 if size == "small" else 6):
        M, N, K, tA, tB, lda, ldb, ldd, a_off, inplace = _draw(rng, size)
        alpha, beta = [(1, 0), (1, 1), (-3, 2), (7, -1)][int(rng.integers(0, 4))]
        inplace = inplace and beta != 0
        got, ref, path = run_i8(M, N, K, tA, tB, alpha, beta, seed=31 * i + block, lda=lda,
                                ldb=ldb, ldd=ldd, a_off=a_off, inplace=inplace)
        say(f"  path: {path}")
        paths.add(path.split(" ")[2] if path.startswith("i8 mfma") else path)
        assert path.startswith("i8 mfma"), path
        assert np.array_equal(got[:M, :N], ref), (M, N, K, tA, tB, alpha, beta, lda, ldb, ldd)
        if not inplace:
            assert np.all(got[:M, N:] == SENTINEL), "kernel wrote past column N"
    say(f"kernels: {sorted(paths)}")


@pytest.mark.parametrize("size,block", [("small", 0), ("small", 1), ("mid", 0), ("mid", 1)])
def test_random_fp8_calls(size, block, monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_PATH", raising=False)
    need_gpu()
    rng = np.random.default_rng(7070 + 10 * block + (size == "mid"))
    for i in range(12 if size == "small" else 6):
        M, N, K, tA, tB, lda, ldb, ldd, a_off, inplace = _draw(rng, size)
        dt = ["f8e4m3", "f8e5m2"][int(rng.integers(0, 2))]
        alpha = float(rng.choice([1.0, -1.5, 0.25]))
        beta = float(rng.choice([0.0, 1.0, -0.5]))
        inplace = inplace and beta != 0.0
        D, D_ref, bound, path = run_fp8(dt, M, N, K, tA, tB, alpha, beta, seed=41 * i + block,
                                        lda=lda, ldb=ldb, ldd=ldd, a_off=a_off, inplace=inplace)
        say(f"  path: {path}")
        assert path.startswith("fp8 " + dt[2:]), path
        rep = oracle.check(D[:M, :N].astype(np.float64), D_ref, bound)
        assert rep["ok"], (dt, M, N, K, tA, tB, alpha, beta, lda, ldb, ldd, rep)
        if not inplace:
            assert np.all(D[:M, N:].view(np.uint32) == D_SENTINEL), "kernel wrote past column N"
