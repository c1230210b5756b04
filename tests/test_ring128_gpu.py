"""GPU parity of the 128x128 direct-to-LDS ring kernel against the oracle.

The kernel stages each operand either straight into LDS or through
registers, for both stored orientations, with edge tiles, K tails and a ring
of five half-slots whose schedule changes with the number of 64-deep K
slices (one slice: prologue only; two: no third slice requested; more: the
ring turns). Every combination is checked elementwise against the oracle,
and the exact cases (permutation and integer inputs) bitwise.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import need_gpu, run

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(monkeypatch):
    need_gpu()
    monkeypatch.delenv("GEMM_FORCE_PATH", raising=False)
    monkeypatch.setenv("GEMM_FORCE_TILE", "t128x128x64")


def _ld(cols, aligned):
    """Leading dimension for a row of `cols` 16-bit values: padded to a 16-byte
    pitch, or one element past it (2-byte pitch: staged through registers)."""
    p = (cols + 7) // 8 * 8
    return p if aligned else p + 1


LAYOUTS = [(0, 1), (0, 0), (1, 1), (1, 0)]
# (A direct-capable pitch, B direct-capable pitch)
MODES = [(True, True), (False, True), (True, False), (False, False)]


@pytest.mark.parametrize("kg", ["shared", "ksplit2", "deep", "pp", "ppdeep"])
@pytest.mark.parametrize("tA,tB", LAYOUTS)
@pytest.mark.parametrize("mode", MODES)
def test_ring_layouts_modes_and_slice_counts(tA, tB, mode, kg, monkeypatch):
    """K from one slice of 64 (prologue only; with two K groups the second
    group then has no slice at all) through two and three slices to several
    turns of the ring, K tails that cut a 16-byte piece (K % 8 != 0) and ones
    that do not; whole tiles and edge tiles on both M and N; one K group per
    workgroup and two; the deep ring (ten half-slots, four slices ahead, both
    operands loaded straight into LDS); the two-group forms (two wave groups
    taking turns, both operands straight into LDS, five or ten half-slots)."""
    monkeypatch.setenv("GEMM_RING_MODE", kg)
    a_al, b_al = mode
    direct_only = kg in ("deep", "pp", "ppdeep")
    if direct_only and mode != (True, True):
        pytest.skip("this form loads both operands straight into LDS")
    seed = 7000 + 97 * LAYOUTS.index((tA, tB)) + 13 * MODES.index(mode) + 1000 * len(kg)
    cases = [(256, 384, 64), (256, 128, 128), (384, 256, 192), (128, 128, 320),
             (300, 260, 72), (136, 200, 1000), (264, 136, 1032), (129, 127, 17)]
    for (M, N, K) in cases:
        for alpha, beta in [(1.0, 0.0), (1.0, 1.0), (-1.5, 0.5)]:
            seed += 1
            lda = _ld(M if tA else K, a_al)
            ldb = _ld(K if tB else N, b_al)
            if direct_only and ((M % 8 and tA) or (N % 8 and not tB) or K % 8):
                continue  # an edge cuts a 16-byte piece: staged, not this form
            cfg = workloads.Config(f"ring{seed}", M, N, K, "bf16" if seed % 2 else "f16", tA, tB,
                                   alpha, beta, "uniform", seed, lda=lda, ldb=ldb,
                                   ldc=N + 3, ldd=N + 3)
            r = run(cfg)
            assert " ring" in r.path and (" ring deep" in r.path) == (kg == "deep") \
                and (" ring ksplit2" in r.path) == (kg == "ksplit2") \
                and (" ring two-group" in r.path) == (kg in ("pp", "ppdeep")) \
                and (" two-group deep" in r.path) == (kg == "ppdeep"), r.path
            r.check()
            r.check_padding_untouched()


@pytest.mark.parametrize("kg", ["shared", "ksplit2", "deep", "pp", "ppdeep"])
@pytest.mark.parametrize("tA,tB", LAYOUTS)
@pytest.mark.parametrize("aligned", [True, False])
def test_ring_permutations_pin_layouts_bitwise(tA, tB, aligned, kg, monkeypatch):
    """P @ X and X @ Q move every element to a known place exactly: a wrong
    swizzle, fragment lane or slot in either staging mode, or a wrong row in
    the K groups' exchange, shows up."""
    if kg in ("deep", "pp", "ppdeep") and not aligned:
        pytest.skip("this form loads both operands straight into LDS")
    monkeypatch.setenv("GEMM_RING_MODE", kg)
    rng = np.random.default_rng(300 + 2 * tA + tB + (8 if aligned else 0))
    M, N, K = 256, 256, 256
    X = torch.tensor(rng.uniform(-1, 1, (M, N)).astype(np.float32)).bfloat16().float().numpy()
    P = np.eye(M, dtype=np.float32)[rng.permutation(M)]
    Q = np.eye(N, dtype=np.float32)[:, rng.permutation(N)]
    for A, B in [(P, X), (X, Q)]:
        As = A.T if tA else A
        Bs = B.T if tB else B
        lda, ldb = _ld(As.shape[1], aligned), _ld(Bs.shape[1], aligned)
        Ap = np.zeros((As.shape[0], lda), np.float32)
        Ap[:, :As.shape[1]] = As
        Bp = np.zeros((Bs.shape[0], ldb), np.float32)
        Bp[:, :Bs.shape[1]] = Bs
        cfg = workloads.Config("ringperm", M, N, K, "bf16", tA, tB, 1.0, 0.0, "uniform", 1,
                               lda=lda, ldb=ldb)
        inp = workloads.make_inputs(cfg, A_src=torch.tensor(Ap), B_src=torch.tensor(Bp))
        r = run(cfg, inp)
        assert " ring" in r.path and (("staged" in r.path) != aligned), r.path
        assert np.array_equal(r.D[:, :N].numpy(), (A @ B).astype(np.float32))


@pytest.mark.parametrize("kg", ["shared", "ksplit2"])
def test_ring_integer_inputs_with_ragged_edges_bitwise(kg, monkeypatch):
    """Integer-valued operands: every partial sum is exact, so D must equal
    the exact product bitwise, here on the ragged shape of the transposed-A
    workload (M = 4097 cuts a 16-byte piece of A's rows; K = 1032)."""
    monkeypatch.setenv("GEMM_RING_MODE", kg)
    rng = np.random.default_rng(5)
    M, N, K = 4097, 1000, 1032
    A = rng.integers(-2, 3, (M, K)).astype(np.float32)
    B = rng.integers(-2, 3, (K, N)).astype(np.float32)
    cfg = workloads.Config("ringint", M, N, K, "f16", 1, 0, 1.0, 0.0, "uniform", 1, lda=M)
    inp = workloads.make_inputs(cfg, A_src=torch.tensor(np.ascontiguousarray(A.T)),
                                B_src=torch.tensor(B))
    r = run(cfg, inp)
    assert " masked staged (A:" in r.path and " ring" in r.path, r.path
    assert np.array_equal(r.D[:, :N].numpy(), (A @ B).astype(np.float32))


@pytest.mark.parametrize("tA,tB", LAYOUTS)
def test_ring_edge_waves_and_inplace(tA, tB, monkeypatch):
    """Edge tiles whose waves hold no or few valid atoms (one row past a
    multiple of 128, a column edge inside a wave's block), C == D, an
    unaligned operand; D untouched outside M x N."""
    seed = 9100 + 10 * LAYOUTS.index((tA, tB))
    for (M, N, K, inplace, pad) in [(4097, 1000, 1032, False, 1), (1000, 4097, 520, True, 0),
                                    (129, 1000, 256, False, 0), (1024, 4100, 200, False, 3)]:
        seed += 1
        lda = (M if tA else K) + pad
        ldb = (K if tB else N) + (8 if seed % 2 else 0)
        ld = N + (0 if inplace else 2)
        cfg = workloads.Config(f"edge{seed}", M, N, K, "f16" if seed % 2 else "bf16", tA, tB,
                               1.5, -0.5 if not inplace else 1.0, "uniform", seed, lda=lda,
                               ldb=ldb, ldc=ld, ldd=ld, inplace=inplace)
        r = run(cfg)
        assert " ring" in r.path, r.path
        r.check()
        r.check_padding_untouched()


@pytest.mark.parametrize("tA,tB", LAYOUTS)
def test_ring_fold_rows_past_the_last_tile_row(tA, tB, monkeypatch):
    """Up to 4 rows past the last whole tile row, computed by that tile
    row's workgroups when that keeps the grid at one tile per CU (16x16x32
    atoms under the tile, A loaded as K pairs and gathered across lanes, B
    from the tile's own slot, the two K groups' sums met through LDS):
    remainders 1, 3 and 4,
    K tails, every epilogue, C == D; elementwise against the oracle on rows
    that cover every tile row and all folded rows; D untouched outside
    M x N. The same shapes with the single-group ring forced take the extra
    tile row instead and must agree."""
    monkeypatch.delenv("GEMM_RING_MODE", raising=False)
    seed = 9700 + 10 * LAYOUTS.index((tA, tB))
    for (M, N, K, alpha, beta, inplace) in [(2049, 2048, 200, 1.0, 0.0, False),
                                            (2051, 2000, 137, 1.5, -0.5, False),
                                            (1028, 4096, 72, 1.0, 1.0, True)]:
        seed += 1
        lda = _ld(M if tA else K, False)  # staged A: the fold applies
        ldb = _ld(K if tB else N, seed % 2 == 0)
        ld = N + (0 if inplace else 4)
        cfg = workloads.Config(f"fold{seed}", M, N, K, "bf16" if seed % 2 else "f16", tA, tB,
                               alpha, beta, "uniform", seed, lda=lda, ldb=ldb, ldc=ld, ldd=ld,
                               inplace=inplace)
        inp = workloads.make_inputs(cfg)
        r = run(cfg, inp)
        nfold = M % 128
        assert f" ring ksplit2 fold({nfold} row" in r.path, r.path
        rows = np.unique(np.concatenate([np.arange(M - 130, M),
                                         np.arange(0, M, 97), np.arange(127, M, 128)]))
        r.check(rows=rows)
        r.check_padding_untouched()
        monkeypatch.setenv("GEMM_RING_MODE", "shared")
        r2 = run(cfg, inp)
        monkeypatch.delenv("GEMM_RING_MODE")
        assert " ring" in r2.path and "fold" not in r2.path, r2.path
        r2.check(rows=rows)


@pytest.mark.parametrize("kg", ["shared", "ksplit2"])
@pytest.mark.parametrize("tA,tB", LAYOUTS)
def test_single_staged_operand_depths_agree_bitwise(tA, tB, kg, monkeypatch):
    """One operand staged through registers: requested three slices ahead
    into two register sets (default) or two slices ahead into one
    (GEMM_STAGE_DEPTH=1). Slice counts of 1 to 6 per K group (the two-set
    loop runs in pairs of iterations), edges on M and N, a K tail; both
    against the oracle and bitwise equal to each other (same sums, same
    order)."""
    monkeypatch.setenv("GEMM_RING_MODE", kg)
    seed = 9900 + 10 * LAYOUTS.index((tA, tB)) + (5 if kg == "shared" else 0)
    # every contiguous dimension a multiple of 8, so only the operand with
    # the odd row pitch is staged
    for (M, N, K) in [(296, 264, 64), (264, 296, 136), (136, 264, 200), (264, 136, 392),
                      (200, 200, 704), (128, 128, 768)]:
        for stage_a in (True, False):
            seed += 1
            lda = _ld(M if tA else K, not stage_a)
            ldb = _ld(K if tB else N, stage_a)
            cfg = workloads.Config(f"depth{seed}", M, N, K, "bf16" if seed % 2 else "f16", tA, tB,
                                   1.5, -0.5, "uniform", seed, lda=lda, ldb=ldb)
            inp = workloads.make_inputs(cfg)
            r2 = run(cfg, inp)
            assert ("staged (A:" in r2.path) == stage_a and " ring" in r2.path, r2.path
            monkeypatch.setenv("GEMM_STAGE_DEPTH", "1")
            r1 = run(cfg, inp)
            monkeypatch.delenv("GEMM_STAGE_DEPTH")
            assert r1.path == r2.path
            assert torch.equal(r1.D, r2.D)
            r2.check()

