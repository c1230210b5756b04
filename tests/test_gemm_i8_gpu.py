"""GPU parity of the int8 -> int32 form against the integer oracle (bit-exact)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import need_gpu, say

pytestmark = pytest.mark.gpu

SENTINEL = -0x21524111  # 0xDEADBEEF as int32: never a result in these cases


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run_i8(M, N, K, tA, tB, alpha, beta, *, seed=0, lda=None, ldb=None, ldd=None, dist=128,
           A=None, B=None, inplace=False, a_off=0):
    import dense_gemm_tile_amd as dgt
    rng = np.random.default_rng(seed)
    lda = lda or (M if tA else K) or 1
    ldb = ldb or (K if tB else N) or 1
    ldd = ldd or N
    a_rows, b_rows = (K if tA else M), (N if tB else K)
    if A is None:
        A = rng.integers(-dist, dist, a_rows * lda).astype(np.int8)
    if B is None:
        B = rng.integers(-dist, dist, b_rows * ldb).astype(np.int8)
    C = rng.integers(-2**31, 2**31, max(M, 1) * ldd).astype(np.int32)
    dev = torch.device("cuda:0")
    a_buf = torch.zeros(a_off + max(A.size, 1), dtype=torch.int8)
    a_buf[a_off:a_off + A.size] = torch.from_numpy(A)
    Ad = a_buf.to(dev)[a_off:]
    Bd = torch.from_numpy(B).to(dev) if B.size else torch.zeros(1, dtype=torch.int8, device=dev)
    Cd = torch.from_numpy(C).to(dev)
    if inplace:
        Dd = Cd
    else:
        Dd = torch.full((max(M, 1) * ldd,), SENTINEL, dtype=torch.int32, device=dev)
    say(f"i8 M={M} N={N} K={K} tA={tA} tB={tB} a={alpha} b={beta} lds={lda},{ldb},{ldd} "
        f"off={a_off} inplace={inplace}")
    dgt.gemm_i8(M, N, K, tA, tB, alpha, beta, Ad, lda, Bd, ldb, Cd if beta != 0 else None, ldd,
                Dd, ldd)
    path = dgt.gemm_last_path()
    torch.cuda.synchronize()
    got = Dd.cpu().numpy().reshape(-1, ldd)
    ref = oracle.gemm_reference_i8(M, N, K, tA, tB, alpha, beta, A, lda, B, ldb, C, ldd)
    return got, ref, path


SHAPES = [(1, 1, 1), (16, 8, 16), (130, 70, 200), (256, 256, 256), (300, 129, 520),
          (513, 65, 130), (64, 200, 31)]


@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 1), (1, 0)])
def test_i8_parity_shapes_layouts_epilogues(tA, tB):
    seed = 0
    for (M, N, K) in SHAPES:
        for alpha, beta in [(1, 0), (1, 1), (-3, 2), (2**31 - 1, -2**31)]:
            seed += 1
            lda = ((M if tA else K) + 15) // 16 * 16
            ldb = ((K if tB else N) + 15) // 16 * 16
            got, ref, path = run_i8(M, N, K, tA, tB, alpha, beta, seed=seed, lda=lda, ldb=ldb,
                                    ldd=N + 3)
            assert path.startswith("i8 mfma"), path
            assert np.array_equal(got[:M, :N], ref), (M, N, K, tA, tB, alpha, beta)
            assert np.all(got[:M, N:] == SENTINEL), "kernel wrote past column N"


@pytest.mark.parametrize("tA,tB", [(0, 1), (1, 0)])
def test_i8_bytewise_staging(tA, tB):
    """Odd pitches and a base one byte past a 16-byte boundary."""
    for (M, N, K), off in [((100, 90, 77), 0), ((257, 130, 300), 1)]:
        lda = (M if tA else K) + 1
        ldb = (K if tB else N) + 3
        got, ref, path = run_i8(M, N, K, tA, tB, 5, -1, seed=M, lda=lda, ldb=ldb, a_off=off)
        assert path.endswith("bytewise staging"), path
        assert np.array_equal(got[:M, :N], ref)


def test_i8_sums_wrap_like_int32():
    # every product is 127*127 (or -128*127): the int32 sums wrap at K = 140000
    M, N, K = 130, 96, 140000
    for a_val in (127, -128):
        A = np.full(M * K, a_val, np.int8)
        B = np.full(N * K, 127, np.int8)
        got, ref, _ = run_i8(M, N, K, 0, 1, 1, 0, A=A, B=B)
        assert np.array_equal(got[:M, :N], ref)
        assert np.all(ref == np.int64(a_val * 127 * K + 2**31) % 2**32 - 2**31)


def test_i8_degenerate_and_inplace():
    for K, alpha in [(0, 1), (64, 0)]:
        got, ref, path = run_i8(70, 50, K, 0, 0, alpha, -3, seed=5)
        assert "D = beta*C" in path and np.array_equal(got[:70, :50], ref)
    got, ref, _ = run_i8(200, 136, 96, 0, 1, 2, 1, seed=6, inplace=True)
    assert np.array_equal(got[:200, :136], ref)


def test_i8_full_size_sampled_rows():
    """8192^3 NT in the launch configuration a benchmark would time; the
    oracle checks rows touching every 128-row tile band."""
    import dense_gemm_tile_amd as dgt
    M = N = K = 8192
    rng = np.random.default_rng(77)
    A = rng.integers(-128, 128, M * K).astype(np.int8)
    B = rng.integers(-128, 128, N * K).astype(np.int8)
    dev = torch.device("cuda:0")
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    Dd = torch.empty(M * N, dtype=torch.int32, device=dev)
    say("i8 8192^3 NT")
    dgt.gemm_i8(M, N, K, 0, 1, 1, 0, Ad, K, Bd, K, None, N, Dd, N)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, M, 128), np.arange(127, M, 128)[::8],
                                     rng.integers(0, M, 8)]))[::4]
    ref = oracle.gemm_reference_i8(M, N, K, 0, 1, 1, 0, A, K, B, K, rows=rows)
    got = Dd.cpu().numpy().reshape(M, N)[rows]
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 1), (1, 0)])
def test_i8_pingpong_whole_tiles_slice_counts(tA, tB):
    """Whole 256x256 tiles take the two-group kernel in every layout (K-
    contiguous operands read with ds_read_b128, M/N-contiguous ones with
    transposed ds_read_b64_tr_b8): K from one 128-byte slice (prologue only)
    to several turns of the five-slot ring, padded leading dimensions, both
    epilogues; bit-exact."""
    seed = 900 + 40 * (2 * tA + tB)
    for K in (128, 256, 384, 512, 640, 1152):
        for alpha, beta in [(1, 0), (-7, 3)]:
            seed += 1
            M, N = 512, 768
            lda = (M if tA else K) + (16 if seed % 2 else 0)
            ldb = (K if tB else N) + (32 if seed % 3 == 0 else 0)
            got, ref, path = run_i8(M, N, K, tA, tB, alpha, beta, seed=seed, lda=lda, ldb=ldb,
                                    ldd=N + 4)
            assert "pingpong" in path and " a16x16x64 " in path, path
            assert np.array_equal(got[:M, :N], ref), (K, alpha, beta)
            assert np.all(got[:M, N:] == SENTINEL)


@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 1), (1, 0)])
def test_i8_pingpong_permutations_pin_layouts(tA, tB):
    """P @ X and X @ Q with int8 X: every element lands in a known place, so a
    wrong lane, swizzle or transposed-read position in either operand shows
    up; bit-exact against the oracle."""
    rng = np.random.default_rng(60 + 2 * tA + tB)
    M = N = K = 256
    X = rng.integers(-128, 128, (M, N)).astype(np.int8)
    P = np.eye(M, dtype=np.int8)[rng.permutation(M)]
    Q = np.eye(N, dtype=np.int8)[:, rng.permutation(N)]
    for Am, Bm in [(P, X), (X, Q)]:
        As = np.ascontiguousarray(Am.T if tA else Am).reshape(-1)
        Bs = np.ascontiguousarray(Bm.T if tB else Bm).reshape(-1)
        got, ref, path = run_i8(M, N, K, tA, tB, 1, 0, A=As, B=Bs)
        assert "pingpong" in path, path
        assert np.array_equal(got[:M, :N], ref)
        assert np.array_equal(got[:M, :N], (Am.astype(np.int32) @ Bm.astype(np.int32)))


def test_i8_inplace_c_is_d_on_both_kernels():
    """C == D with a general epilogue on the two-group kernel (whole 256x256
    tiles, two layouts) and on the 128x128 kernel (a ragged shape),
    bit-exact."""
    got, ref, path = run_i8(512, 768, 640, 0, 1, -3, 2, seed=930, inplace=True)
    assert "pingpong" in path, path
    assert np.array_equal(got[:512, :768], ref)
    got, ref, path = run_i8(512, 768, 640, 1, 0, 5, -1, seed=931, inplace=True)
    assert "pingpong" in path, path
    assert np.array_equal(got[:512, :768], ref)
    got, ref, path = run_i8(300, 200, 520, 1, 0, 5, -1, seed=932, inplace=True)
    assert "pingpong" not in path, path
    assert np.array_equal(got[:300, :200], ref)


@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 1), (1, 0)])
def test_i8_pingpong_edge_tiles(tA, tB):
    """Shapes that do not tile 256x256 (K a multiple of 16, N of 4, the
    contiguous dimension of an M/N-contiguous operand of 16) take the
    two-group kernel with edge tiles: pieces outside the operands read as
    zeros, C and D accessed inside M x N only. Edges on M and N, K tails of
    16 to 112 bytes past the last whole slice, padded leading dimensions,
    both epilogues, C == D; bit-exact, D's padding untouched."""
    seed = 1200 + 40 * (2 * tA + tB)
    for (M, N, K) in [(608, 528, 400), (1040, 784, 272), (528, 784, 144), (272, 1040, 1040)]:
        for alpha, beta in [(1, 0), (-7, 3)]:
            seed += 1
            lda = (M if tA else K) + (16 if seed % 2 else 0)
            ldb = (K if tB else N) + (32 if seed % 3 == 0 else 0)
            got, ref, path = run_i8(M, N, K, tA, tB, alpha, beta, seed=seed, lda=lda, ldb=ldb,
                                    ldd=N + 4)
            assert "pingpong masked" in path, path
            assert np.array_equal(got[:M, :N], ref), (M, N, K, alpha, beta)
            assert np.all(got[:M, N:] == SENTINEL)
    got, ref, path = run_i8(608, 528, 400, tA, tB, -3, 2, seed=seed + 1, inplace=True)
    assert "pingpong masked" in path, path
    assert np.array_equal(got[:608, :528], ref)


@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 1), (1, 0)])
def test_i8_pingpong_elementwise_cd(tA, tB):
    """C and D rows not 16-byte aligned (odd leading dimension) or N % 4 != 0
    (where B is K-contiguous): the two-group kernel with edge tiles reads C
    and writes D element by element; both epilogues, C == D; bit-exact, D's
    padding untouched."""
    seed = 1500 + 40 * (2 * tA + tB)
    cases = [(608, 528, 400, 529), (1040, 784, 272, 787)]
    if tB:
        cases += [(528, 1030, 144, 1030), (1040, 1025, 272, 1027)]
    for (M, N, K, ldd) in cases:
        for alpha, beta in [(1, 0), (-7, 3)]:
            seed += 1
            lda = (M if tA else K) + (16 if seed % 2 else 0)
            got, ref, path = run_i8(M, N, K, tA, tB, alpha, beta, seed=seed, lda=lda, ldd=ldd)
            assert path.endswith("pingpong masked elementwise C/D"), path
            assert np.array_equal(got[:M, :N], ref), (M, N, K, ldd, alpha, beta)
            assert np.all(got[:M, N:] == SENTINEL)
    got, ref, path = run_i8(608, 528, 400, tA, tB, -3, 2, seed=seed + 1, ldd=531, inplace=True)
    assert path.endswith("pingpong masked elementwise C/D"), path
    assert np.array_equal(got[:608, :528], ref)

