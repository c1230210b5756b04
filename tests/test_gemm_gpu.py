"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bar: |D - D_ref| <= 2e-3*(|alpha|*(|A|@|B|) + |beta*C|) + 1e-6 elementwise;
bitwise equality where the exact result is representable and every partial
sum is exact (integer, identity and permutation inputs).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import D_SENTINEL, need_gpu, run, sample_rows, say

pytestmark = pytest.mark.gpu

C = workloads.CONFIGS


@pytest.fixture(autouse=True)
def _gpu(monkeypatch):
    need_gpu()
    monkeypatch.delenv("GEMM_FORCE_PATH", raising=False)
    monkeypatch.delenv("GEMM_FORCE_TILE", raising=False)


def _dt(cfg):
    return workloads.DTYPE_CODE[cfg.dtype]


# ----------------------------------------------- the five workloads ---------

@pytest.mark.parametrize("name", ["atom16x8x16", "gemm512", "ragged4097x1000x1032_tn"])
def test_workload_parity_full(name):
    r = run(C[name])
    r.check()
    r.check_padding_untouched()
    assert r.path.startswith("mfma "), r.path
    if name == "ragged4097x1000x1032_tn":
        # row 4096 folded into the last whole tile row (256 tiles, two K groups)
        assert " ring ksplit2 fold(1 row) masked staged (A: row pitch 8194 B" in r.path, r.path


@pytest.mark.parametrize("name", ["gemm4096_inplace", "gemm8192_nt"])
def test_workload_parity_full_size_sampled(name):
    """Full size in the launch configuration the benchmark times; the oracle
    checks rows that touch every 256-row tile band (all columns), and one
    element at a random position inside every 64x64 block of D, so every
    output tile and every wave's sub-tile is checked somewhere."""
    cfg = C[name]
    r = run(cfg)
    assert r.path.startswith("mfma t256x256x64"), r.path
    r.check(rows=sample_rows(cfg.M, 256, 1))
    r.check_elements(block=64, seed=cfg.seed)
    assert np.all(np.isfinite(r.D.numpy()))


def test_f32_operand_workload_full_size_sampled():
    """The float32-operand workload (4096^3 NT, rounded to bf16 on the GPU) in
    the launch configuration the benchmark times, against the oracle's own
    rounding on rows that touch every 256-row tile band."""
    cfg = workloads.EXTRA_CONFIGS["gemm4096_f32in_nt"]
    r = run(cfg)
    assert r.path == "mfma t256x256x64 w2x4 a32x32x16 NT epi=beta0 pingpong f32->bf16", r.path
    r.check(rows=sample_rows(cfg.M, 256, 1))
    assert np.all(np.isfinite(r.D.numpy()))


def test_ragged_workload_on_mfma_with_aligned_pitch():
    """Same ragged shape with A's rows padded to a 16-byte pitch: the masked
    matrix-core path must agree with the oracle too."""
    cfg = workloads.with_shape(C["ragged4097x1000x1032_tn"], lda=4104)
    r = run(cfg)
    assert r.path.startswith("mfma ") and " masked" in r.path, r.path
    r.check()


@pytest.mark.parametrize("name", ["atom16x8x16", "gemm512", "ragged4097x1000x1032_tn"])
def test_workload_parity_forced_fma(name, monkeypatch):
    monkeypatch.setenv("GEMM_FORCE_PATH", "fma")
    r = run(C[name])
    assert r.path.startswith("fma "), r.path
    r.check()


@pytest.mark.parametrize("name", ["gemm4096_inplace", "gemm8192_nt"])
def test_full_size_workload_forced_fma_sampled(name, monkeypatch):
    """The two full-size workloads on the VALU-FMA path: sampled rows touching
    every 512-row band, and one element inside every 256x256 block."""
    monkeypatch.setenv("GEMM_FORCE_PATH", "fma")
    cfg = C[name]
    r = run(cfg)
    assert r.path.startswith("fma "), r.path
    r.check(rows=sample_rows(cfg.M, 512, 1))
    r.check_elements(block=256, seed=cfg.seed + 1)


# ---------------------------------------------- tiled shape sweep -----------

SHAPES = [(16, 8, 16), (1, 1, 1), (32, 32, 16), (48, 40, 24), (64, 64, 64), (100, 130, 70),
          (257, 129, 200), (128, 256, 96), (300, 17, 33), (5, 300, 8), (513, 65, 130),
          (256, 256, 256), (96, 160, 1000), (64, 96, 768)]
TILES = ["t16x16x64", "t64x64x64", "t128x128x64", "t256x256x64", "t32x32x64k4", "t32x32x64k8",
         "t64x64x64k4"]


def _on_tile(path, tile):
    """The forced tile ran, or for the 256x256 tile (whole tiles with 16-byte
    rows only, on the two-group kernel) a call that needs masking or register
    staging ran on 128x128 tiles."""
    if tile == "t256x256x64" and path.startswith("mfma t128x128x64"):
        return any(k in path for k in (" masked", "staged (", "narrow staging ("))
    # the 64x64 four-group tile runs whole tiles of K % 256 == 0 only: other
    # calls take the tile chosen without it (checked on the host)
    if tile == "t64x64x64k4" and not path.startswith("mfma " + tile):
        return path.startswith("mfma ")
    return path.startswith("mfma " + tile)


def _pad8(x):
    return (x + 7) // 8 * 8


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiled_shapes(tile, dtype, monkeypatch):
    monkeypatch.setenv("GEMM_FORCE_TILE", tile)
    seed = 2000
    for (M, N, K) in SHAPES:
        for tA, tB in [(0, 0), (0, 1), (1, 0), (1, 1)]:
            for alpha, beta in [(1.0, 0.0), (1.0, 1.0), (1.5, 0.5)]:
                seed += 1
                # padded leading dims keep rows 16-byte aligned (matrix-core path)
                lda = _pad8(M if tA else K) + (8 if seed % 3 == 0 else 0)
                ldb = _pad8(K if tB else N)
                ldd = N + (seed % 5)
                cfg = workloads.Config(f"sweep{seed}", M, N, K, dtype, tA, tB, alpha, beta,
                                       "uniform", seed, lda=lda, ldb=ldb, ldc=ldd, ldd=ldd)
                r = run(cfg)
                assert _on_tile(r.path, tile), r.path
                r.check()
                r.check_padding_untouched()


def _ld_with_width(x, vw):
    """Smallest leading dimension >= x whose 2-byte row pitch allows loads of
    exactly vw elements (8: 16-byte aligned, 4: 8-byte, 2: 4-byte, 1: 2-byte)."""
    ld = x
    while True:
        w = 8
        while w > 1 and (ld * 2) % (2 * w):
            w //= 2
        if w == vw:
            return ld
        ld += 1


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiled_shapes_narrow_staging(tile, dtype, monkeypatch):
    """Operands whose row pitch or base address is not a multiple of 16 bytes
    stay on the matrix cores, read with 8-, 4- or 2-byte loads: pitches of
    each width, bases 4 or 2 bytes past a 16-byte boundary, one or both
    operands, every layout."""
    monkeypatch.setenv("GEMM_FORCE_TILE", tile)
    seed = 5000
    # (A width, B width, A offset, B offset in elements)
    modes = [(1, 8, 0, 1), (8, 4, 0, 0), (2, 1, 0, 0), (4, 2, 2, 0)]
    for (M, N, K) in SHAPES[1::2] + [(512, 512, 192)]:
        for tA, tB in [(0, 0), (0, 1), (1, 0), (1, 1)]:
            seed += 1
            wa, wb, a_off, b_off = modes[seed % 4]
            lda = _ld_with_width(M if tA else K, wa)
            ldb = _ld_with_width(K if tB else N, wb)
            cfg = workloads.Config(f"narrow{seed}", M, N, K, dtype, tA, tB, 1.5, -0.5,
                                   "uniform", seed, lda=lda, ldb=ldb)
            r = run(cfg, a_off=a_off, b_off=b_off)
            assert _on_tile(r.path, tile), r.path
            # the general kernels read such operands in narrow pieces; the
            # 128x128 ring kernel stages them through registers
            assert ("narrow staging (" in r.path) != (" ring" in r.path and "staged (" in r.path), \
                r.path
            r.check()
            r.check_padding_untouched()


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("dtype", ["f32_f16", "f32_bf16"])
def test_tiled_shapes_f32_operands(tile, dtype, monkeypatch):
    """float32 A and B rounded to f16/bf16 (as staged: through registers on
    the 128x128 ring kernel, on the masked kernel at the other tiles; as read
    from LDS on whole NT tiles): every layout, general epilogue, aligned and
    8-/4-byte pitches, bases 4 bytes past a 16-byte boundary; NaN in the
    padding is never read."""
    monkeypatch.setenv("GEMM_FORCE_TILE", tile)
    seed = 6000
    for (M, N, K) in SHAPES[::2] + [(512, 256, 192)]:
        for tA, tB in [(0, 0), (0, 1), (1, 0), (1, 1)]:
            seed += 1
            mode = seed % 3
            lda = (M if tA else K) + (0, 1, 2)[mode]
            ldb = (K if tB else N) + (3, 0, 2)[mode]
            a_off = 1 if mode == 1 else 0  # elements of 4 bytes
            cfg = workloads.Config(f"f32op{seed}", M, N, K, dtype, tA, tB, 1.5, -0.5,
                                   "uniform", seed, lda=lda, ldb=ldb)
            r = run(cfg, a_off=a_off)
            assert _on_tile(r.path, tile) and (" f32->" + dtype[4:]) in r.path, r.path
            r.check()
            r.check_padding_untouched()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_f32_operands_equal_prerounded_16bit_bitwise(dtype):
    """Rounding inside the staging is the same rounding torch applies, and
    the rest of the path is the same kernel: D must match bitwise."""
    cfg32 = workloads.Config("f32eq", 300, 200, 136, "f32_" + dtype, 0, 1, 1.0, 0.0,
                             "normal", 91)
    inp32 = workloads.make_inputs(cfg32)
    r32 = run(cfg32, inp32)
    cfg16 = workloads.Config("f32eq16", 300, 200, 136, dtype, 0, 1, 1.0, 0.0, "normal", 91)
    r16 = run(cfg16, workloads.make_inputs(cfg16, A_src=inp32.A_src, B_src=inp32.B_src))
    assert r32.path.replace(" f32->" + dtype, "") == r16.path, (r32.path, r16.path)
    assert torch.equal(r32.D, r16.D)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_f32_operands_pingpong(dtype, monkeypatch):
    """Whole 256x256 tiles of float32 operands take the two-group kernel in
    every layout, which rounds each fragment as it reads it from LDS: one
    slice of 32, two, an odd count, and many; every epilogue; padded leading
    dimensions; against the oracle."""
    monkeypatch.setenv("GEMM_FORCE_TILE", "t256x256x64")
    seed = 6500
    for (tA, tB) in [(0, 1), (0, 0), (1, 1), (1, 0)]:
        for K in (32, 64, 96, 1056):
            for alpha, beta in [(1.0, 0.0), (1.0, 1.0), (1.5, -0.5)]:
                seed += 1
                pad = 4 * (seed % 3)
                cfg = workloads.Config(f"f32pp{seed}", 512, 256, K, "f32_" + dtype, tA, tB, alpha,
                                       beta, "uniform", seed, ldd=256 + 4 * (seed % 2),
                                       lda=(512 if tA else K) + pad,
                                       ldb=(K if tB else 256) + pad)
                r = run(cfg)
                assert "pingpong f32->" + dtype in r.path and "masked" not in r.path, r.path
                r.check()
                r.check_padding_untouched()
    # M or N edges and K tails (K-contiguous operands: K a multiple of 4; an
    # M/N-contiguous operand: its M or N): the same kernel with edge tiles,
    # pieces past the operands reading as zeros; C == D
    for (tA, tB, M, N, K) in [(0, 0, 300, 260, 48), (1, 1, 516, 200, 40), (0, 1, 301, 299, 44),
                              (1, 0, 260, 516, 37), (1, 0, 8, 4, 3)]:
        for alpha, beta in [(1.0, 0.0), (-1.5, 0.5)]:
            seed += 1
            ip = beta != 0.0
            cfg = workloads.Config(f"f32pp{seed}", M, N, K, "f32_" + dtype, tA, tB, alpha, beta,
                                   "uniform", seed, ldc=N + (0 if ip else 4),
                                   ldd=N + (0 if ip else 4), inplace=ip)
            r = run(cfg)
            assert r.path.endswith("pingpong masked f32->" + dtype), r.path
            r.check()
            r.check_padding_untouched()
    # a contiguous dimension cut inside a 16-byte piece, or 8-byte rows: the
    # 128x128 ring kernel, both operands staged and rounded in registers
    for (tA, tB, K, ldb) in [(0, 1, 42, None), (0, 1, 64, 66)]:
        seed += 1
        cfg = workloads.Config(f"f32pp{seed}", 512, 256, K, "f32_" + dtype, tA, tB, 1.0, 0.0,
                               "uniform", seed, ldb=ldb)
        r = run(cfg)
        assert " ring" in r.path and "staged (A, B: float32" in r.path and "pingpong" not in r.path, \
            r.path
        r.check()


@pytest.mark.parametrize("mode", ["shared", "ksplit2"])
@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_f32_ring_rounding_bitwise(dtype, tA, tB, mode, monkeypatch):
    """float32 operands on the 128x128 ring kernel are rounded in registers
    and written where 16-bit pieces would go: D must equal, bitwise, D of the
    same ring form fed the operands the oracle rounds (ties of both parities,
    values one ulp off a tie, subnormals of the 16-bit format), in every
    layout, with M/N edges that cut a 16-byte piece and a K tail."""
    monkeypatch.setenv("GEMM_FORCE_TILE", "t128x128x64")
    monkeypatch.setenv("GEMM_RING_MODE", mode)
    rng = np.random.default_rng(70 + 2 * tA + tB)
    M, N, K = 300, 260, 200
    code = 0 if dtype == "f16" else 1
    A32 = _tie_heavy_f32((K, M) if tA else (M, K), dtype, rng)
    B32 = _tie_heavy_f32((N, K) if tB else (K, N), dtype, rng)

    def oracle_rounded(x):
        bits = oracle.round_f32_bits(x.numpy().reshape(-1), code)
        return torch.tensor(oracle.decode_bits(bits, code).astype(np.float32).reshape(x.shape))

    cfg32 = workloads.Config("f32ring", M, N, K, "f32_" + dtype, tA, tB, 1.0, 0.0, "uniform", 1)
    r32 = run(cfg32, workloads.make_inputs(cfg32, A_src=A32, B_src=B32))
    assert " ring" in r32.path and "staged (A, B: float32" in r32.path, r32.path
    cfg16 = workloads.Config("f32ring16", M, N, K, dtype, tA, tB, 1.0, 0.0, "uniform", 1)
    r16 = run(cfg16, workloads.make_inputs(cfg16, A_src=oracle_rounded(A32),
                                           B_src=oracle_rounded(B32)))
    assert " ring" in r16.path and (" ring ksplit2" in r16.path) == (mode == "ksplit2"), r16.path
    assert torch.equal(r32.D, r16.D)
    r32.check()


def _tie_heavy_f32(shape, dtype, rng):
    """float32 values that stress rounding to the 16-bit format: exact ties
    between two neighbours (both parities), one float32 ulp either side of a
    tie, subnormals of the 16-bit format, and plain random values."""
    n = int(np.prod(shape))
    if dtype == "bf16":
        hi = rng.integers(0x3C00, 0x4080, n, dtype=np.uint32)   # |x| about 2^-7 .. 4
        hi |= rng.integers(0, 2, n, dtype=np.uint32) << 15       # sign
        low = np.choose(rng.integers(0, 4, n), [np.full(n, 0x8000), np.full(n, 0x8001),
                                                 np.full(n, 0x7FFF), rng.integers(0, 0x10000, n)])
        bits = (hi << 16) | low.astype(np.uint32)
        sub = rng.random(n) < 0.1  # bf16 subnormals: float32 exponent field 0
        bits[sub] = (bits[sub] & 0x8000FFFF) | (rng.integers(1, 0x80, sub.sum()).astype(np.uint32) << 16)
        x = bits.view(np.float32)
    else:
        h = (rng.standard_normal(n) * 2.0).astype(np.float16)
        nxt = np.nextafter(h, np.float16(np.inf))
        mid = (h.astype(np.float32) + nxt.astype(np.float32)) / 2  # exact in float32
        x = np.choose(rng.integers(0, 4, n),
                      [mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf)),
                       rng.standard_normal(n).astype(np.float32)])
        sub = rng.random(n) < 0.1  # f16 subnormals and ties between them
        x[sub] = (rng.integers(-1023, 1024, sub.sum()) * 2.0 ** -25).astype(np.float32)
    return torch.tensor(x.astype(np.float32).reshape(shape))


@pytest.mark.parametrize("shape", [(256, 512, 192), (264, 520, 200)])
@pytest.mark.parametrize("tA,tB", [(0, 1), (0, 0), (1, 1), (1, 0)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_f32_pingpong_rounding_bitwise(dtype, tA, tB, shape, monkeypatch):
    """In-register rounding of the two-group kernel against the oracle's
    rounding, in every layout (M/N-contiguous operands are read down their
    float32 K-rows), whole tiles and edge tiles: D from float32 operands must
    equal, bitwise, D of the 16-bit kernel fed the operands the oracle rounds
    (same tile, same sum order; zeros past the operands add nothing)."""
    monkeypatch.setenv("GEMM_FORCE_TILE", "t256x256x64")
    rng = np.random.default_rng(44 + 2 * tA + tB + shape[2])
    M, N, K = shape  # both sides on the two-group design
    A32 = _tie_heavy_f32((K, M) if tA else (M, K), dtype, rng)
    B32 = _tie_heavy_f32((N, K) if tB else (K, N), dtype, rng)
    code = 0 if dtype == "f16" else 1

    def oracle_rounded(x):
        bits = oracle.round_f32_bits(x.numpy().reshape(-1), code)
        return torch.tensor(oracle.decode_bits(bits, code).astype(np.float32).reshape(x.shape))

    cfg32 = workloads.Config("f32tie", M, N, K, "f32_" + dtype, tA, tB, 1.0, 0.0, "uniform", 1)
    r32 = run(cfg32, workloads.make_inputs(cfg32, A_src=A32, B_src=B32))
    assert r32.path.endswith(("pingpong f32->" + dtype, "pingpong masked f32->" + dtype)), r32.path
    cfg16 = workloads.Config("f32tie16", M, N, K, dtype, tA, tB, 1.0, 0.0, "uniform", 1)
    r16 = run(cfg16, workloads.make_inputs(cfg16, A_src=oracle_rounded(A32),
                                           B_src=oracle_rounded(B32)))
    # Same tile and slice order; the 16-bit kernel multiplies on 16x16x32
    # atoms, the float32-operand one on 32x32x16, whose sums agree bit for
    # bit (each adds its K-values to the accumulator in the same 16-wide
    # steps), so D must still be equal bitwise.
    assert r32.path.replace(" f32->" + dtype, "") == \
        r16.path.replace("a16x16x32", "a32x32x16"), (r32.path, r16.path)
    assert torch.equal(r32.D, r16.D)
    r32.check()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiled_shapes_fma(dtype, monkeypatch):
    monkeypatch.setenv("GEMM_FORCE_PATH", "fma")
    seed = 3000
    for (M, N, K) in SHAPES:
        for tA, tB in [(0, 0), (0, 1), (1, 0), (1, 1)]:
            seed += 1
            cfg = workloads.Config(f"fsweep{seed}", M, N, K, dtype, tA, tB, 2.0, -1.0,
                                   "uniform", seed,
                                   lda=(M if tA else K) + seed % 3, ldb=(K if tB else N) + 1)
            r = run(cfg)
            assert r.path.startswith("fma "), r.path
            r.check()


# ---------------------------------------------------- exact cases -----------

def _exact_case(dtype, tA, tB, M, N, K, A, B, path):
    """Run with the given op(A) [M,K] and op(B) [K,N] float matrices whose
    products and partial sums are exact; require bitwise equality."""
    As = A.T if tA else A
    Bs = B.T if tB else B
    cfg = workloads.Config(f"exact-{dtype}-{tA}{tB}", M, N, K, dtype, tA, tB, 1.0, 0.0,
                           "uniform", 1, lda=As.shape[1], ldb=Bs.shape[1])
    inp = workloads.make_inputs(cfg, A_src=torch.tensor(As, dtype=torch.float32),
                                B_src=torch.tensor(Bs, dtype=torch.float32))
    r = run(cfg, inp)
    assert r.path.startswith(path), r.path
    D_ref, _ = r.reference()
    got = r.D[:, :N].numpy()
    assert np.array_equal(got, D_ref.astype(np.float32)), \
        np.argwhere(got != D_ref.astype(np.float32))[:5]


PATHS = ["mfma", "fma"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_exact_integer_inputs(path, dtype, tA, tB, monkeypatch):
    monkeypatch.setenv("GEMM_FORCE_PATH", path)
    rng = np.random.default_rng(7 + tA + 2 * tB)
    M, N, K = 264, 272, 520
    A = rng.integers(-2, 3, (M, K)).astype(np.float32)
    B = rng.integers(-2, 3, (K, N)).astype(np.float32)
    _exact_case(dtype, tA, tB, M, N, K, A, B, path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_exact_permutations_pin_lane_ownership(path, tA, tB, monkeypatch):
    """P @ X and X @ Q move every element to a known place exactly, so any
    wrong lane/row/column ownership in a fragment or accumulator shows up."""
    monkeypatch.setenv("GEMM_FORCE_PATH", path)
    rng = np.random.default_rng(11 + tA + 2 * tB)
    for tile in (["t256x256x64", "t64x64x64", "t64x64x64k4", "t16x16x64"] if path == "mfma"
                 else [None]):
        if tile:
            monkeypatch.setenv("GEMM_FORCE_TILE", tile)
        M = K = N = 256
        X = rng.uniform(-1, 1, (M, N)).astype(np.float32)
        X = torch.tensor(X).bfloat16().float().numpy()  # values exact in bf16
        P = np.eye(M, dtype=np.float32)[rng.permutation(M)]
        Q = np.eye(N, dtype=np.float32)[:, rng.permutation(N)]
        _exact_case("bf16", tA, tB, M, N, K, P, X, path)
        _exact_case("bf16", tA, tB, M, N, K, X, Q, path)
        I = np.eye(K, dtype=np.float32)
        _exact_case("bf16", tA, tB, M, N, K, X, I, path)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_exact_k_tails(tile, dtype, monkeypatch):
    """The last K step runs only the sub-steps holding valid K-values; with
    16x16x32 atoms a valid part of at most 16 finishes on 16x16x16. Integer
    inputs make every order exact, so the result must match bitwise."""
    monkeypatch.setenv("GEMM_FORCE_TILE", tile)
    rng = np.random.default_rng(21)
    for K in (1, 8, 16, 17, 24, 32, 40, 48, 56, 63, 80, 112):
        for tA, tB in [(0, 0), (1, 1)] if K % 2 else [(0, 1), (1, 0)]:
            M, N = 48, 40
            A = rng.integers(-2, 3, (M, K)).astype(np.float32)
            B = rng.integers(-2, 3, (K, N)).astype(np.float32)
            As = A.T if tA else A
            Bs = B.T if tB else B
            lda = (As.shape[1] + 7) // 8 * 8
            ldb = (Bs.shape[1] + 7) // 8 * 8
            cfg = workloads.Config(f"ktail{K}", M, N, K, dtype, tA, tB, 1.0, 0.0, "uniform", 1,
                                   lda=lda, ldb=ldb)
            Ap = np.zeros((As.shape[0], lda), np.float32)
            Ap[:, :As.shape[1]] = As
            Bp = np.zeros((Bs.shape[0], ldb), np.float32)
            Bp[:, :Bs.shape[1]] = Bs
            inp = workloads.make_inputs(cfg, A_src=torch.tensor(Ap), B_src=torch.tensor(Bp))
            r = run(cfg, inp)
            assert _on_tile(r.path, tile), r.path
            # the general kernels on 16x16x32 atoms (a forced tile may fall back)
            atom16 = r.path.startswith(("mfma t16x16x64 ", "mfma t64x64x64 "))
            assert (" k16-tail" in r.path) == (atom16 and 1 <= K % 32 <= 16), r.path
            got = r.D[:, :N].numpy()
            assert np.array_equal(got, (A @ B).astype(np.float32)), (K, tA, tB)


def test_exact_ones_closed_form():
    M, N, K = 300, 200, 2048
    cfg = workloads.Config("ones", M, N, K, "bf16", 0, 1, 1.0, 0.0, "uniform", 1)
    inp = workloads.make_inputs(cfg, A_src=torch.ones(M, K), B_src=torch.ones(N, K))
    r = run(cfg, inp)
    assert np.all(r.D.numpy() == float(K))


@pytest.mark.parametrize("kg", [4, 8])
def test_k_split_is_deterministic_and_exact(kg, monkeypatch):
    """The K groups' partial sums are added in a fixed order: two runs agree
    bitwise; with integer inputs every partial sum is exact, so D is the exact
    product. K = 2120 leaves the groups unequal numbers of steps and a ragged tail."""
    monkeypatch.setenv("GEMM_FORCE_TILE", f"t32x32x64k{kg}")
    M, N, K = 512, 512, 2120
    cfg = workloads.Config("ksplit", M, N, K, "bf16", 0, 0, 1.5, 0.5, "normal", 77)
    r1 = run(cfg)
    r2 = run(cfg)
    assert f" ksplit{kg} masked" in r1.path, r1.path
    assert torch.equal(r1.D, r2.D)
    r1.check()
    rng = np.random.default_rng(5)
    A = rng.integers(-3, 4, (M, K)).astype(np.float32)
    B = rng.integers(-3, 4, (K, N)).astype(np.float32)
    for tA, tB in [(0, 0), (1, 1)]:
        cfg = workloads.Config("ksplit_int", M, N, K, "f16", tA, tB, 1.0, 0.0, "uniform", 1)
        inp = workloads.make_inputs(cfg, A_src=torch.tensor(A.T.copy() if tA else A),
                                    B_src=torch.tensor(B.T.copy() if tB else B))
        r = run(cfg, inp)
        assert f" ksplit{kg}" in r.path, r.path
        assert np.array_equal(r.D[:, :N].numpy(), (A @ B).astype(np.float32)), (tA, tB)


def test_huge_pitch_64bit_addressing():
    """A row pitch whose byte offsets across one tile pass 2^31 (A with
    2^24 + 8 elements per row: an 8 GiB extent, of which only the M x K
    elements are written and read) takes the masked kernel's 64-bit
    addressing; D must match the oracle on the packed operand."""
    import dense_gemm_tile_amd as dgt
    dev = torch.device("cuda:0")
    M, N, K = 256, 192, 256
    lda = (1 << 24) + 8
    cfg = workloads.Config("hugepitch", M, N, K, "bf16", 0, 0, 1.0, 0.0, "uniform", 97)
    inp = workloads.make_inputs(cfg)
    say(f"huge pitch M={M} N={N} K={K} lda={lda}")
    Abig = torch.empty((M - 1) * lda + K, dtype=torch.bfloat16, device=dev)
    Abig.as_strided((M, K), (lda, 1)).copy_(inp.A.to(dev))
    B = inp.B.to(dev)
    D = torch.full((M, N), float("nan"), device=dev)
    dgt.gemm(M, N, K, "bf16", 0, 0, 1.0, 0.0, Abig, lda, B, N, None, N, D, N)
    path = dgt.gemm_last_path()
    torch.cuda.synchronize()
    assert " masked" in path, path
    D_ref, bound = oracle.gemm_reference(M, N, K, 1, 0, 0, 1.0, 0.0,
                                         workloads.bits_u16(inp.A).reshape(-1), K,
                                         workloads.bits_u16(inp.B).reshape(-1), N)
    rep = oracle.check(D.cpu().numpy().astype(np.float64), D_ref, bound)
    del Abig
    torch.cuda.empty_cache()
    assert rep["ok"], rep


# ----------------------------------------------- epilogue and aliasing ------

def test_inplace_equals_separate_buffers_bitwise():
    base = workloads.Config("ip", 512, 384, 320, "bf16", 0, 0, 1.0, 1.0, "normal", 77)
    inp = workloads.make_inputs(base)
    sep = run(base, inp)
    ip = run(workloads.with_shape(base, inplace=True), inp)
    assert torch.equal(sep.D[:, :384], ip.D[:, :384])
    sep.check()


def test_epilogue_forms_are_consistent_bitwise():
    """alpha=1,beta=1 equals (alpha=1,beta=0) + C in float32; alpha=2 equals 2x."""
    base = workloads.Config("epi", 320, 288, 192, "f16", 1, 0, 1.0, 0.0, "uniform", 78,
                            lda=320)
    inp = workloads.make_inputs(base, want_c=True)
    d0 = run(base, inp).D
    d1 = run(workloads.with_shape(base, beta=1.0), inp).D
    assert torch.equal(d1, d0 + inp.C)
    d2 = run(workloads.with_shape(base, alpha=2.0), inp).D
    assert torch.equal(d2, 2.0 * d0)


@pytest.mark.parametrize("path", PATHS)
def test_beta_zero_never_reads_c(path, monkeypatch):
    monkeypatch.setenv("GEMM_FORCE_PATH", path)
    cfg = workloads.Config("nanc", 200, 136, 96, "bf16", 0, 0, 1.0, 0.0, "uniform", 79)
    inp = workloads.make_inputs(cfg, C=torch.full((200, 136), float("nan")))
    r = run(cfg, inp)  # a NaN-filled C is passed, and must not be read
    assert np.all(np.isfinite(r.D.numpy()))
    r.check()


def test_k_zero_and_alpha_zero():
    import dense_gemm_tile_amd as dgt
    dev = torch.device("cuda:0")
    M, N = 70, 90
    Cm = torch.rand(M, N, device=dev) * 2 - 1
    D = torch.full((M, N), 5.0, device=dev)
    say("K=0 beta=-0.5")
    dgt.gemm(M, N, 0, "f16", 0, 0, 1.0, -0.5, None, 1, None, N, Cm, N, D, N,
             stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(D, -0.5 * Cm)
    say("alpha=0 beta=0")
    A = torch.full((M, 8), float("nan"), device=dev, dtype=torch.float16)
    B = torch.full((8, N), float("nan"), device=dev, dtype=torch.float16)
    dgt.gemm(M, N, 8, "f16", 0, 0, 0.0, 0.0, A, 8, B, N, None, N, D, N,
             stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(D, torch.zeros_like(D))


def test_errors_launch_nothing():
    import dense_gemm_tile_amd as dgt
    dev = torch.device("cuda:0")
    D = torch.full((8, 8), 3.0, device=dev)
    A = torch.ones(8, 8, device=dev, dtype=torch.float16)
    st = dgt.gemm_status(8, 8, 8, 0, 0, 0, 1.0, 0.0, A, 8, A, 8, None, 8, D, 4,
                         stream=torch.cuda.current_stream())
    assert st == dgt.GEMM_ERR_INVALID_ARG
    st = dgt.gemm_status(8, 8, 8, 0, 0, 0, 1.0, 0.0, A, 8, D, 8, None, 8, D, 8,
                         stream=torch.cuda.current_stream())
    assert st == dgt.GEMM_ERR_ALIAS
    torch.cuda.synchronize()
    assert torch.equal(D, torch.full((8, 8), 3.0, device=dev))


def test_deterministic_repeat_and_side_stream():
    cfg = workloads.Config("det", 1024, 768, 1536, "bf16", 0, 1, 1.0, 0.0, "normal", 80)
    inp = workloads.make_inputs(cfg)
    a = run(cfg, inp).D
    b = run(cfg, inp).D
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = run(cfg, inp, stream=s).D
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("layout", [(0, 1), (0, 0), (1, 1), (1, 0)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_pingpong_path_slice_counts(dtype, layout, monkeypatch):
    """Whole 256x256 tiles take the two-group kernel with direct loads, for
    K-contiguous operands (ds_read_b128 fragments) and M/N-contiguous ones
    (transposed ds_read_b64_tr_b16 fragments); K from one slice of 64
    (prologue only) through two (no load in the loop) to several turns of the
    five-slot ring; padded leading dimensions."""
    monkeypatch.setenv("GEMM_FORCE_TILE", "t256x256x64")
    tA, tB = layout
    seed = 4000 + 100 * (2 * tA + tB)
    for K in (64, 128, 192, 256, 320, 384, 448, 640, 1024):
        for alpha, beta in [(1.0, 0.0), (1.0, 1.0), (-0.5, 2.0)]:
            seed += 1
            M, N = 512, 768
            lda = (M if tA else K) + (8 if seed % 2 else 0)
            ldb = (K if tB else N) + (16 if seed % 3 == 0 else 0)
            cfg = workloads.Config(f"pp{seed}", M, N, K, dtype, tA, tB, alpha, beta,
                                   "uniform", seed, lda=lda, ldb=ldb, ldd=N + 4, ldc=N + 4)
            r = run(cfg)
            assert "pingpong" in r.path, r.path
            r.check()
            r.check_padding_untouched()


def test_pingpong_grid_walks_tiles_unevenly():
    """Whole 256x256 tiles run on a grid of at most 256 workgroups, each
    walking tiles blockIdx.x, + 256, ...: with 289 tiles the first 33
    workgroups take two tiles and the rest one. Rows touching every tile band
    and one element in every 64x64 block against the oracle; C == D."""
    M = N = 17 * 256
    cfg = workloads.Config("ppwalk", M, N, 256, "bf16", 0, 1, 1.0, 1.0, "uniform", 4352,
                           inplace=True)
    r = run(cfg)
    assert r.path == "mfma t256x256x64 w2x4 a16x16x32 NT epi=acc+c pingpong", r.path
    r.check(rows=sample_rows(M, 256, 1))
    r.check_elements(block=64, seed=cfg.seed)


PP_EDGE_SHAPES = {
    # (M, N, K, C == D); every layout's contiguous dimensions are multiples of 8
    "any": [(520, 264, 1000, False), (264, 776, 72, True), (8, 520, 8, False),
            (768, 40, 200, False), (1032, 1288, 136, True), (256, 256, 24, False)],
    # edges that only the layout's M/N-contiguous operands allow
    (0, 1): [(301, 299, 136, False)],
    (0, 0): [(301, 264, 200, True)],
    (1, 1): [(264, 299, 200, False)],
    (1, 0): [(264, 264, 137, False), (264, 520, 3, True)],
}


@pytest.mark.parametrize("layout", [(0, 1), (0, 0), (1, 1), (1, 0)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_pingpong_edge_tiles(dtype, layout, monkeypatch):
    """Edge tiles on the two-group kernel: M and N edges inside a wave's
    block and ones that leave whole waves or a whole wave group outside,
    K tails inside a 64-deep slice and K shorter than one slice (pieces past
    the operand read as zeros; each 16-byte piece is whole because the
    operand's contiguous dimension is a multiple of 8), every epilogue,
    C == D, padded leading dimensions; D untouched outside M x N."""
    monkeypatch.setenv("GEMM_FORCE_TILE", "t256x256x64")
    tA, tB = layout
    seed = 4700 + 100 * (2 * tA + tB) + (50 if dtype == "bf16" else 0)
    for (M, N, K, inplace) in PP_EDGE_SHAPES["any"] + PP_EDGE_SHAPES[layout]:
        for alpha, beta in [(1.0, 0.0), (1.0, 1.0), (-1.5, 0.5)]:
            seed += 1
            lda = _pad8(M if tA else K) + (8 if seed % 2 else 0)
            ldb = _pad8(K if tB else N) + (16 if seed % 3 == 0 else 0)
            ip = inplace and beta != 0.0  # C == D needs an epilogue that reads C
            ld = N + (0 if ip else 4)
            cfg = workloads.Config(f"ppedge{seed}", M, N, K, dtype, tA, tB, alpha, beta,
                                   "uniform", seed, lda=lda, ldb=ldb, ldc=ld, ldd=ld,
                                   inplace=ip)
            r = run(cfg)
            assert r.path.startswith("mfma t256x256x64") and r.path.endswith(" pingpong masked"), \
                r.path
            r.check()
            r.check_padding_untouched()


@pytest.mark.parametrize("layout", [(0, 1), (0, 0), (1, 1), (1, 0)])
def test_pingpong_edge_tiles_integer_inputs_bitwise(layout, monkeypatch):
    """Integer-valued operands make every partial sum exact: with edge tiles
    on M, N and a K tail, D must equal the exact product bitwise (zeros read
    past the operands add nothing; a piece read from the wrong place or a
    lost slice shows up)."""
    monkeypatch.setenv("GEMM_FORCE_TILE", "t256x256x64")
    tA, tB = layout
    rng = np.random.default_rng(61 + 2 * tA + tB)
    M, N, K = 520, 776, 1000
    A = rng.integers(-2, 3, (M, K)).astype(np.float32)
    B = rng.integers(-2, 3, (K, N)).astype(np.float32)
    _exact_case("bf16", tA, tB, M, N, K, A, B, "mfma t256x256x64")


@pytest.mark.parametrize("shape", [(4000, 4000, 4096, 0, 1, 0.0), (4000, 3904, 4100, 1, 0, 1.0)])
def test_pingpong_edge_tiles_full_size_sampled(shape):
    """A 256-tile grid of edge tiles at full size, planned without forcing:
    4000^2 x 4096 NT, and TN with an N edge and a K tail reading C; rows that
    touch every 256-row tile band and one element in every 64x64 block."""
    M, N, K, tA, tB, beta = shape
    cfg = workloads.Config(f"ppedge{M}x{N}x{K}", M, N, K, "bf16", tA, tB, 1.0, beta, "uniform",
                           77 + tA)
    r = run(cfg)
    assert r.path.startswith("mfma t256x256x64") and r.path.endswith(" pingpong masked"), r.path
    r.check(rows=sample_rows(cfg.M, 256, 1))
    r.check_elements(block=64, seed=cfg.seed)


SPLIT_CASES = [
    # (M, N, K, dtype, tA, tB, alpha, beta, C == D): remainder rows and
    # columns, rows only, columns only; every layout; float32 operands
    (4097, 4097, 256, "bf16", 0, 1, 1.5, -0.5, False),
    (4128, 4100, 192, "f16", 0, 0, 1.0, 1.0, True),
    (4104, 4096, 136, "bf16", 1, 0, 1.0, 0.0, False),
    (4096, 4127, 320, "f16", 1, 1, -2.0, 0.5, False),
    (4097, 4100, 96, "f32_bf16", 0, 1, 1.0, 0.0, False),
    (4200, 4224, 200, "bf16", 0, 1, 1.0, 1.0, True),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}_{c[3]}_{c[4]}{c[5]}")
def test_split_past_a_multiple_of_the_tile(case, monkeypatch):
    """Up to 128 rows and columns past the last whole 256x256 tile that would
    add a round of tiles: the call runs as the whole tiles, the remainder
    rows and the remainder columns, three launches on one stream. Rows that
    touch every tile band (the remainder rows included) against the oracle
    over all columns, one element in every 64x64 block, D untouched outside
    M x N; the same path from gemm_validate."""
    monkeypatch.delenv("GEMM_FORCE_TILE", raising=False)
    M, N, K, dtype, tA, tB, alpha, beta, inplace = case
    pad8 = lambda x: (x + 7) // 8 * 8  # 16-byte rows for every operand
    lda = pad8(M if tA else K)
    ldb = pad8(K if tB else N)
    ld = N + (0 if inplace else 4)
    cfg = workloads.Config(f"split{M}x{N}x{K}", M, N, K, dtype, tA, tB, alpha, beta, "uniform",
                           M + N + K, lda=lda, ldb=ldb, ldc=ld, ldd=ld, inplace=inplace)
    r = run(cfg)
    assert r.path.startswith("split core "), r.path
    assert (f"; rows {M % 256}x{N}:" in r.path) == (M % 256 > 0), r.path
    assert (f"; cols {M - M % 256}x{N % 256}:" in r.path) == (N % 256 > 0), r.path
    rows = np.unique(np.concatenate([sample_rows(M, 256, 1), np.arange(M - 40, M)]))
    r.check(rows=rows)
    if not dtype.startswith("f32"):  # the per-element oracle takes 16-bit operands
        r.check_elements(block=64, seed=cfg.seed)
    r.check_padding_untouched()
    import dense_gemm_tile_amd as dgt
    st = dgt.gemm_validate(M, N, K, dtype, tA, tB, alpha, beta, 1 << 32, lda, 2 << 32, ldb,
                           (3 << 32) if beta else None, ld, (3 << 32) if inplace else 4 << 32,
                           ld)
    assert st == dgt.GEMM_OK and dgt.gemm_last_path() == r.path, dgt.gemm_last_path()


@pytest.mark.parametrize("layout", [(0, 1), (0, 0), (1, 1)])
def test_wide_and_scalar_epilogues_agree(layout):
    """Whole tiles store D with 16-byte accesses when D (and C) allow it and
    element by element otherwise; both must match the oracle, and each other
    bitwise (same accumulators, same epilogue arithmetic)."""
    import dense_gemm_tile_amd as dgt
    tA, tB = layout
    M, N, K = 512, 512, 256
    dev = torch.device("cuda:0")
    base = workloads.Config("epiw", M, N, K, "bf16", tA, tB, 1.5, -0.5, "uniform", 90)
    inp = workloads.make_inputs(base)
    wide = run(base, inp)
    # D one float past a 16-byte boundary, C with an odd leading dimension
    lda, ldb, _, _ = base.lds()
    A, B = inp.A.to(dev), inp.B.to(dev)
    Cp = torch.zeros((M, N + 1), device=dev)
    Cp[:, :N] = inp.C.to(dev)
    Dbuf = torch.full((M * N + 1,), float("nan"), device=dev)
    say(f"scalar epilogue {layout}")
    dgt.gemm(M, N, K, "bf16", tA, tB, 1.5, -0.5, A, lda, B, ldb, Cp, N + 1,
             Dbuf.data_ptr() + 4, N, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    scalar = Dbuf[1:].reshape(M, N).cpu()
    assert torch.equal(wide.D[:, :N], scalar)
    wide.check()
