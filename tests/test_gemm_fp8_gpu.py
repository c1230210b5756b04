"""GPU parity of the 8-bit float forms (OCP E4M3, E5M2) against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import D_SENTINEL, need_gpu, say

pytestmark = pytest.mark.gpu

FMT = {"f8e4m3": 4, "f8e5m2": 5}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run_fp8(dt, M, N, K, tA, tB, alpha, beta, *, seed=0, lda=None, ldb=None, ldd=None,
            a_off=0, A=None, B=None, inplace=False):
    import dense_gemm_tile_amd as dgt
    fmt = FMT[dt]
    lda = lda or (M if tA else K) or 1
    ldb = ldb or (K if tB else N) or 1
    ldd = ldd or N
    if A is None:
        A, B = workloads.make_fp8_inputs(M, N, K, tA, tB, fmt, seed, lda=lda, ldb=ldb)
    gen = torch.Generator("cpu").manual_seed(seed + 1)
    C = (torch.rand((max(M, 1), ldd), generator=gen) * 2 - 1)
    dev = torch.device("cuda:0")
    a_buf = torch.zeros(a_off + A.numel(), dtype=torch.uint8)
    a_buf[a_off:] = A.reshape(-1)
    Ad = a_buf.to(dev)[a_off:]
    Bd = B.reshape(-1).to(dev)
    Cd = C.to(dev)
    if inplace:  # D is C itself (same pointer and leading dimension)
        Dd = Cd
    else:
        Dd = torch.empty((max(M, 1), ldd), dtype=torch.float32, device=dev)
        Dd.view(torch.int32).fill_(int(np.uint32(D_SENTINEL).view(np.int32)))
    say(f"{dt} M={M} N={N} K={K} tA={tA} tB={tB} a={alpha} b={beta} lds={lda},{ldb},{ldd} "
        f"off={a_off} inplace={inplace}")
    dgt.gemm(M, N, K, dt, tA, tB, alpha, beta, Ad, lda, Bd, ldb, Cd if beta != 0 else None,
             ldd, Dd, ldd)
    path = dgt.gemm_last_path()
    torch.cuda.synchronize()
    D = Dd.cpu().numpy()
    D_ref, bound = oracle.gemm_reference(M, N, K, fmt, tA, tB, alpha, beta,
                                         A.numpy().reshape(-1), lda, B.numpy().reshape(-1), ldb,
                                         C.numpy().reshape(-1), ldd)
    return D, D_ref, bound, path


SHAPES = [(1, 1, 1), (16, 8, 16), (130, 70, 200), (256, 256, 256), (300, 129, 520),
          (64, 200, 31)]


@pytest.mark.parametrize("dt", ["f8e4m3", "f8e5m2"])
@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 1), (1, 0)])
def test_fp8_parity_shapes_layouts(dt, tA, tB):
    seed = 10 * FMT[dt] + 2 * tA + tB
    for (M, N, K) in SHAPES:
        for alpha, beta in [(1.0, 0.0), (0.25, -1.5)]:
            seed += 100
            lda = ((M if tA else K) + 15) // 16 * 16
            ldb = ((K if tB else N) + 15) // 16 * 16
            D, D_ref, bound, path = run_fp8(dt, M, N, K, tA, tB, alpha, beta, seed=seed,
                                            lda=lda, ldb=ldb, ldd=N + 2)
            assert path.startswith("fp8 " + dt[2:]), path
            rep = oracle.check(D[:M, :N].astype(np.float64), D_ref, bound)
            assert rep["ok"], (dt, M, N, K, tA, tB, rep)
            pad = D[:M, N:].view(np.uint32)
            assert np.all(pad == D_SENTINEL), "kernel wrote past column N"


@pytest.mark.parametrize("dt", ["f8e4m3", "f8e5m2"])
def test_fp8_bytewise_staging(dt):
    D, D_ref, bound, path = run_fp8(dt, 257, 130, 300, 1, 0, 1.0, 0.0, seed=3, lda=258,
                                    ldb=133, a_off=1)
    assert path.endswith("bytewise staging"), path
    assert oracle.check(D[:257, :130].astype(np.float64), D_ref, bound)["ok"]


def test_fp8_exact_small_integers():
    """Codes of small integers (exact in both formats), products and sums
    exact in f32: the result must match bitwise; pins each lane's rows,
    columns and K range."""
    rng = np.random.default_rng(4)
    M, N, K = 96, 80, 192
    for dt, table in [("f8e4m3", {-2: 0xC0, -1: 0xB8, 0: 0x00, 1: 0x38, 2: 0x40}),
                      ("f8e5m2", {-2: 0xC0, -1: 0xBC, 0: 0x00, 1: 0x3C, 2: 0x40})]:
        av = rng.integers(-2, 3, (M, K))
        bv = rng.integers(-2, 3, (N, K))
        enc = np.vectorize(lambda v: table[int(v)])
        A = torch.from_numpy(enc(av).astype(np.uint8))
        B = torch.from_numpy(enc(bv).astype(np.uint8))
        assert np.array_equal(oracle.decode_fp8(A.numpy(), FMT[dt]), av)
        D, D_ref, _, _ = run_fp8(dt, M, N, K, 0, 1, 1.0, 0.0, A=A, B=B)
        assert np.array_equal(D[:M, :N], (av @ bv.T).astype(np.float32))


def test_fp8_full_size_sampled_rows():
    """8192^3 NT E4M3 in the launch configuration a benchmark would time."""
    import dense_gemm_tile_amd as dgt
    M = N = K = 8192
    A, B = workloads.make_fp8_inputs(M, N, K, 0, 1, 4, 1008)
    dev = torch.device("cuda:0")
    Ad, Bd = A.to(dev), B.to(dev)
    D = torch.empty((M, N), dtype=torch.float32, device=dev)
    say("f8e4m3 8192^3 NT")
    dgt.gemm(M, N, K, "f8e4m3", 0, 1, 1.0, 0.0, Ad, K, Bd, K, None, N, D, N)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 4095, 4096, 8191])
    D_ref, bound = oracle.gemm_reference(M, N, K, 4, 0, 1, 1.0, 0.0, A.numpy().reshape(-1), K,
                                         B.numpy().reshape(-1), K, rows=rows)
    assert oracle.check(D[rows].cpu().numpy().astype(np.float64), D_ref, bound)["ok"]


@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 1), (1, 0)])
@pytest.mark.parametrize("dt", ["f8e4m3", "f8e5m2"])
def test_fp8_pingpong_whole_tiles_slice_counts(dt, tA, tB):
    """Whole 256x256 tiles take the two-group kernel in every layout: K from
    one 128-byte slice to several turns of the five-slot ring, padded leading
    dimensions."""
    seed = 950 + 20 * (2 * tA + tB)
    for K in (128, 256, 384, 640, 1152):
        seed += 1
        M, N = 512, 768
        lda = (M if tA else K) + (16 if seed % 2 else 0)
        ldb = (K if tB else N) + 32
        D, D_ref, bound, path = run_fp8(dt, M, N, K, tA, tB, 0.5, -1.0, seed=seed, lda=lda,
                                        ldb=ldb, ldd=N + 4)
        assert "pingpong" in path and " a16x16x128 " in path, path
        assert oracle.check(D[:M, :N].astype(np.float64), D_ref, bound)["ok"], (dt, K)
        assert np.all(D[:M, N:].view(np.uint32) == D_SENTINEL)


@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 1), (1, 0)])
def test_fp8_pingpong_exact_small_integers(tA, tB):
    """Small integers are exact in E4M3 and their sums exact in f32, so D
    must equal the integer product bitwise in every layout."""
    rng = np.random.default_rng(8 + 2 * tA + tB)
    M, N, K = 256, 512, 384
    table = {-2: 0xC0, -1: 0xB8, 0: 0x00, 1: 0x38, 2: 0x40}
    av = rng.integers(-2, 3, (M, K))
    bv = rng.integers(-2, 3, (N, K))
    enc = np.vectorize(lambda v: table[int(v)])
    A = torch.from_numpy(np.ascontiguousarray(enc(av.T if tA else av).astype(np.uint8)))
    B = torch.from_numpy(np.ascontiguousarray(enc(bv if tB else bv.T).astype(np.uint8)))
    D, _, _, path = run_fp8("f8e4m3", M, N, K, tA, tB, 1.0, 0.0, A=A, B=B)
    assert "pingpong" in path, path
    assert np.array_equal(D[:M, :N], (av @ bv.T).astype(np.float32))


@pytest.mark.parametrize("dt", ["f8e4m3", "f8e5m2"])
def test_fp8_inplace_c_is_d(dt):
    """D may be C itself: each element of C is read before the same lane
    writes D there. Both the 128x128 kernel (a ragged shape) and the
    two-group kernel (whole 256x256 tiles, two layouts) are run with C == D and a
    general epilogue, against the oracle on the original C."""
    for (M, N, K, tA, tB) in [(300, 129, 520, 1, 0), (512, 768, 384, 0, 1),
                              (512, 768, 384, 1, 0)]:
        D, D_ref, bound, path = run_fp8(dt, M, N, K, tA, tB, 1.5, -0.75, seed=970 + M + tA,
                                        inplace=True)
        if M == 512:
            assert "pingpong" in path, path
        else:
            assert "pingpong" not in path, path
        rep = oracle.check(D[:M, :N].astype(np.float64), D_ref, bound)
        assert rep["ok"], (dt, M, N, K, rep)


@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 1), (1, 0)])
@pytest.mark.parametrize("dt", ["f8e4m3", "f8e5m2"])
def test_fp8_pingpong_edge_tiles(dt, tA, tB):
    """Shapes that do not tile 256x256 take the two-group kernel with edge
    tiles (see the int8 test): edges on M and N, K tails, padded leading
    dimensions, a general epilogue and C == D; against the oracle, D's
    padding untouched; and small integers, exact in E4M3 with exact f32
    sums, bitwise."""
    seed = 1300 + 20 * (2 * tA + tB)
    for (M, N, K) in [(608, 528, 400), (1040, 784, 272), (272, 1040, 1040)]:
        seed += 1
        lda = (M if tA else K) + (16 if seed % 2 else 0)
        ldb = (K if tB else N) + 32
        D, D_ref, bound, path = run_fp8(dt, M, N, K, tA, tB, 0.5, -1.0, seed=seed, lda=lda,
                                        ldb=ldb, ldd=N + 4)
        assert "pingpong masked" in path, path
        assert oracle.check(D[:M, :N].astype(np.float64), D_ref, bound)["ok"], (dt, M, N, K)
        assert np.all(D[:M, N:].view(np.uint32) == D_SENTINEL)
    D, D_ref, bound, path = run_fp8(dt, 608, 528, 400, tA, tB, 1.5, -0.75, seed=seed + 1,
                                    inplace=True)
    assert "pingpong masked" in path, path
    assert oracle.check(D[:608, :528].astype(np.float64), D_ref, bound)["ok"]
    if dt == "f8e4m3":
        rng = np.random.default_rng(18 + 2 * tA + tB)
        M, N, K = 528, 784, 272
        table = {-2: 0xC0, -1: 0xB8, 0: 0x00, 1: 0x38, 2: 0x40}
        av = rng.integers(-2, 3, (M, K))
        bv = rng.integers(-2, 3, (N, K))
        enc = np.vectorize(lambda v: table[int(v)])
        A = torch.from_numpy(np.ascontiguousarray(enc(av.T if tA else av).astype(np.uint8)))
        B = torch.from_numpy(np.ascontiguousarray(enc(bv if tB else bv.T).astype(np.uint8)))
        D, _, _, path = run_fp8("f8e4m3", M, N, K, tA, tB, 1.0, 0.0, A=A, B=B)
        assert "pingpong masked" in path, path
        assert np.array_equal(D[:M, :N], (av @ bv.T).astype(np.float32))


@pytest.mark.parametrize("dt", ["f8e4m3", "f8e5m2"])
@pytest.mark.parametrize("tA,tB", [(0, 1), (1, 0)])
def test_fp8_pingpong_elementwise_cd(dt, tA, tB):
    """Odd leading dimensions of C and D, or N % 4 != 0: the two-group kernel
    with edge tiles reads C and writes D element by element; a general
    epilogue and C == D; against the oracle, D's padding untouched."""
    seed = 1700 + 20 * (2 * tA + tB) + FMT[dt]
    cases = [(608, 528, 400, 529)] + ([(1040, 1025, 272, 1027)] if tB else [(1040, 784, 272, 785)])
    for (M, N, K, ldd) in cases:
        seed += 1
        D, D_ref, bound, path = run_fp8(dt, M, N, K, tA, tB, 0.5, -1.0, seed=seed, ldd=ldd)
        assert path.endswith("pingpong masked elementwise C/D"), path
        assert oracle.check(D[:M, :N].astype(np.float64), D_ref, bound)["ok"], (dt, M, N, K)
        assert np.all(D[:M, N:].view(np.uint32) == D_SENTINEL)
    D, D_ref, bound, path = run_fp8(dt, 608, 528, 400, tA, tB, 1.5, -0.75, seed=seed + 1,
                                    ldd=531, inplace=True)
    assert path.endswith("pingpong masked elementwise C/D"), path
    assert oracle.check(D[:608, :528].astype(np.float64), D_ref, bound)["ok"]

