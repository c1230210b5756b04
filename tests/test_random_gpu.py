"""Seeded random calls against the oracle, across the planner's choices.

Shapes, layouts, element types, leading dimensions (16-byte rows or not),
alpha/beta and C == D are drawn from a fixed seed, so every run checks the
same calls; the planner picks the kernel (general, ring, two-group, split),
and each result must pass the oracle's bound. The large cases sit just past
multiples of 256 and are checked on sampled rows over all columns.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import need_gpu, run, sample_rows

pytestmark = pytest.mark.gpu

DTYPES = ["f16", "bf16", "f32_f16", "f32_bf16"]


def _draw(rng, size):
    if size == "small":
        M, N, K = (int(x) for x in rng.integers(1, [700, 700, 1200]))
    elif size == "medium":
        M, N = (int(x) for x in rng.integers(700, [2600, 2600]))
        K = int(rng.integers(64, 1300))
    else:
        M = 4096 + int(rng.integers(0, 140))
        N = 4096 + int(rng.integers(0, 140))
        K = int(rng.choice([64, 136, 256, 512]))
    dtype = DTYPES[int(rng.integers(0, len(DTYPES)))]
    tA, tB = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    q = 4 if dtype.startswith("f32") else 8  # elements per 16-byte piece
    pad = lambda x: (x + q - 1) // q * q
    lda = M if tA else K
    ldb = K if tB else N
    lda = pad(lda) if rng.random() < 0.7 else lda + int(rng.integers(0, 3))
    ldb = pad(ldb) if rng.random() < 0.7 else ldb + int(rng.integers(0, 3))
    alpha = float(rng.choice([1.0, -1.5, 0.25]))
    beta = float(rng.choice([0.0, 1.0, -0.5]))
    inplace = beta != 0.0 and rng.random() < 0.3
    ld = N + (0 if inplace else int(rng.integers(0, 5)))
    return M, N, K, dtype, tA, tB, alpha, beta, lda, ldb, ld, inplace


@pytest.mark.parametrize("block", range(4))
def test_random_small_calls(block, monkeypatch):
    for var in ("GEMM_FORCE_PATH", "GEMM_FORCE_TILE", "GEMM_RING_MODE", "GEMM_STAGE_DEPTH"):
        monkeypatch.delenv(var, raising=False)
    need_gpu()
    rng = np.random.default_rng(4242 + block)
    for i in range(20):
        M, N, K, dtype, tA, tB, alpha, beta, lda, ldb, ld, inplace = _draw(rng, "small")
        cfg = workloads.Config(f"rand{block}_{i}", M, N, K, dtype, tA, tB, alpha, beta,
                               "uniform", 100 * block + i, lda=lda, ldb=ldb, ldc=ld, ldd=ld,
                               inplace=inplace)
        r = run(cfg)
        r.check()
        r.check_padding_untouched()


@pytest.mark.parametrize("block", range(2))
def test_random_medium_calls(block, monkeypatch):
    """Grids of tens to hundreds of 128x128 tiles (ring, two-group and
    partial-grid 256x256 forms), checked on sampled rows over all columns."""
    for var in ("GEMM_FORCE_PATH", "GEMM_FORCE_TILE", "GEMM_RING_MODE", "GEMM_STAGE_DEPTH"):
        monkeypatch.delenv(var, raising=False)
    need_gpu()
    rng = np.random.default_rng(6161 + block)
    for i in range(10):
        M, N, K, dtype, tA, tB, alpha, beta, lda, ldb, ld, inplace = _draw(rng, "medium")
        cfg = workloads.Config(f"randM{block}_{i}", M, N, K, dtype, tA, tB, alpha, beta,
                               "uniform", 500 + 10 * block + i, lda=lda, ldb=ldb, ldc=ld, ldd=ld,
                               inplace=inplace)
        r = run(cfg)
        rows = np.unique(np.concatenate([sample_rows(M, 128, 1, seed=i), np.arange(M - 4, M)]))
        r.check(rows=rows)
        r.check_padding_untouched()


@pytest.mark.parametrize("block", range(2))
def test_random_large_calls(block, monkeypatch):
    for var in ("GEMM_FORCE_PATH", "GEMM_FORCE_TILE", "GEMM_RING_MODE", "GEMM_STAGE_DEPTH"):
        monkeypatch.delenv(var, raising=False)
    need_gpu()
    rng = np.random.default_rng(5151 + block)
    for i in range(4):
        M, N, K, dtype, tA, tB, alpha, beta, lda, ldb, ld, inplace = _draw(rng, "large")
        cfg = workloads.Config(f"randL{block}_{i}", M, N, K, dtype, tA, tB, alpha, beta,
                               "uniform", 700 + 10 * block + i, lda=lda, ldb=ldb, ldc=ld, ldd=ld,
                               inplace=inplace)
        r = run(cfg)
        rows = np.unique(np.concatenate([sample_rows(M, 256, 1, seed=i), np.arange(M - 8, M)]))
        r.check(rows=rows)
        r.check_padding_untouched()


TILES = ["t16x16x64", "t64x64x64", "t128x128x64", "t256x256x64", "t32x32x64k4", "t32x32x64k8",
         "t64x64x64k4"]


@pytest.mark.parametrize("tile", TILES)
def test_random_calls_on_each_tile(tile, monkeypatch):
    """The same draws with the tile forced, so every tile's kernels (whole,
    masked, staged, K-split) meet shapes the planner would not give them."""
    for var in ("GEMM_FORCE_PATH", "GEMM_RING_MODE", "GEMM_STAGE_DEPTH"):
        monkeypatch.delenv(var, raising=False)
    monkeypatch.setenv("GEMM_FORCE_TILE", tile)
    need_gpu()
    rng = np.random.default_rng(3131 + TILES.index(tile))
    for i in range(8):
        M, N, K, dtype, tA, tB, alpha, beta, lda, ldb, ld, inplace = _draw(rng, "small")
        cfg = workloads.Config(f"randT{tile}_{i}", M, N, K, dtype, tA, tB, alpha, beta,
                               "uniform", 900 + 10 * TILES.index(tile) + i, lda=lda, ldb=ldb,
                               ldc=ld, ldd=ld, inplace=inplace)
        r = run(cfg)
        r.check()
        r.check_padding_untouched()


def test_random_calls_forced_fma(monkeypatch):
    """The same draws on the VALU-FMA fallback (16-bit operands; it has no
    float32-operand form), which must meet the same bound."""
    for var in ("GEMM_FORCE_TILE", "GEMM_RING_MODE", "GEMM_STAGE_DEPTH"):
        monkeypatch.delenv(var, raising=False)
    monkeypatch.setenv("GEMM_FORCE_PATH", "fma")
    need_gpu()
    rng = np.random.default_rng(2727)
    for i in range(12):
        M, N, K, dtype, tA, tB, alpha, beta, lda, ldb, ld, inplace = _draw(rng, "small")
        dtype = dtype[4:] if dtype.startswith("f32_") else dtype  # 16-bit operands only
        cfg = workloads.Config(f"randF_{i}", M, N, K, dtype, tA, tB, alpha, beta,
                               "uniform", 1000 + i, lda=lda, ldb=ldb, ldc=ld, ldd=ld,
                               inplace=inplace)
        r = run(cfg)
        assert r.path.startswith("fma"), r.path
        r.check()
        r.check_padding_untouched()
