"""Host-side tests of the C-ABI library: exports, argument checks, path choice
and the tile scheduler. Nothing here launches a kernel or needs a GPU; pointer
arguments are fake addresses that the library only compares."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    so = os.path.join(ROOT, "dense_gemm_tile_amd", "libdense_gemm_tile_amd.so")
    if not os.path.exists(so):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_dgt_build", os.path.join(ROOT, "dense_gemm_tile_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import dense_gemm_tile_amd as dgt
    return dgt


def _declared_symbols():
    names = []
    for h in os.listdir(os.path.join(ROOT, "include")):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            names += re.findall(r"GEMM_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)
    return names


def test_library_exports_every_declared_symbol(lib):
    names = _declared_symbols()
    assert {"gemm", "gemm_validate", "gemm_last_error", "gemm_last_path",
            "gemm_tile_order", "gemm_i8", "gemm_i8_validate"} <= set(names)
    so = lib.LIB_PATH
    out = subprocess.run(["nm", "-D", "--defined-only", so], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    # nothing but the C ABI is exported from our own code
    ours = {n for n in exported if n.startswith(("gemm", "_ZN3dgt"))}
    assert ours == set(names)


# Fake, suitably aligned device addresses: never dereferenced on the host.
A0, B0, C0, D0 = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def _v(lib, M=64, N=64, K=64, dtype=0, tA=0, tB=0, alpha=1.0, beta=0.0, A=A0, lda=None,
       B=B0, ldb=None, C=C0, ldc=None, D=D0, ldd=None):
    lda = lda if lda is not None else (M if tA else K)
    ldb = ldb if ldb is not None else (K if tB else N)
    ldc = ldc if ldc is not None else N
    ldd = ldd if ldd is not None else N
    return lib.gemm_validate(M, N, K, dtype, tA, tB, alpha, beta, A, lda, B, ldb, C, ldc, D, ldd)


def test_valid_call_selects_mfma(lib):
    assert _v(lib) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("mfma ")
    assert lib.gemm_last_error() == ""


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), 1), (dict(N=-5), 1), (dict(K=-2), 1),
    (dict(dtype=6), 2), (dict(dtype=-1), 2),
    (dict(lda=63), 1), (dict(tA=1, lda=63), 1), (dict(ldb=63), 1), (dict(tB=1, ldb=63), 1),
    (dict(ldd=63), 1), (dict(beta=1.0, ldc=63), 1),
    (dict(D=0), 1), (dict(A=0), 1), (dict(B=0), 1), (dict(beta=0.5, C=0), 1),
    (dict(D=D0 + 2), 1), (dict(beta=1.0, C=C0 + 2), 1), (dict(A=A0 + 1), 1),
    (dict(M=1 << 31), 2),
])
def test_argument_errors(lib, kw, code):
    assert _v(lib, **kw) == code
    assert lib.gemm_last_error() != ""


def test_ld_check_is_not_needed_for_unread_c(lib):
    # beta == 0: C is not read, so ldc and C itself are ignored
    assert _v(lib, beta=0.0, C=0, ldc=0) == lib.GEMM_OK


def test_alias_rules(lib):
    nbytes_d = 64 * 64 * 4
    assert _v(lib, beta=1.0, C=D0, ldc=64, D=D0, ldd=64) == lib.GEMM_OK  # exact in-place
    assert _v(lib, beta=1.0, C=D0, ldc=128, D=D0, ldd=64) == lib.GEMM_ERR_ALIAS
    assert _v(lib, beta=1.0, C=D0 + 64, D=D0) == lib.GEMM_ERR_ALIAS
    assert _v(lib, beta=1.0, C=D0 + nbytes_d, D=D0) == lib.GEMM_OK  # adjacent, no overlap
    assert _v(lib, A=D0 + 1024, D=D0) == lib.GEMM_ERR_ALIAS
    assert _v(lib, B=D0 - 64, D=D0) == lib.GEMM_ERR_ALIAS
    assert _v(lib, B=D0 - 64 * 64 * 2, D=D0) == lib.GEMM_OK  # B ends where D begins
    # C overlapping D is fine when C is not read
    assert _v(lib, beta=0.0, C=D0 + 4, D=D0) == lib.GEMM_OK


def test_empty_and_degenerate_calls(lib):
    assert _v(lib, M=0, A=0, B=0, D=0) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("noop")
    assert _v(lib, N=0, A=0, B=0, D=0, ldb=1, ldd=1) == lib.GEMM_OK
    assert _v(lib, N=0, A=0, B=0, D=0) == lib.GEMM_ERR_INVALID_ARG  # ld must be >= 1
    assert _v(lib, K=0, A=0, B=0, beta=0.5, lda=1) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("scale")
    assert _v(lib, alpha=0.0, A=0, B=0, beta=2.0) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("scale")
    assert _v(lib, K=0, A=0, B=0, beta=0.0, C=0, lda=1) == lib.GEMM_OK


def test_unaligned_pitch_stays_on_mfma_with_narrow_staging(lib):
    # transposed f16 A with lda = 4097: an 8194-byte row pitch. 128x128 tiles
    # run on the ring kernel, which stages A through registers.
    st = _v(lib, M=4097, N=1000, K=1032, tA=1, lda=4097, alpha=2.0, beta=-1.0)
    assert st == lib.GEMM_OK
    path = lib.gemm_last_path()
    # (row 4096 is folded into the last whole tile row: 256 tiles instead of
    # 264, one per CU, on two K groups)
    assert path == ("mfma t128x128x64 w2x2 a32x32x16 TN epi=general ring ksplit2 fold(1 row) "
                    "masked staged (A: row pitch 8194 B is not a multiple of 16 B)"), path
    # same shape with a 16-byte pitch: A is still staged (M = 4097 cuts its
    # contiguous dimension off a multiple of 8), B is loaded straight into LDS
    assert _v(lib, M=4097, N=1000, K=1032, tA=1, lda=4104) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" ring ksplit2 fold(1 row) masked staged (A: M % 8 != 0)")
    # up to 4 rows fold, and only where that brings the grid to one tile per
    # CU
    assert _v(lib, M=4100, N=1000, K=1032, tA=1, lda=4101) == lib.GEMM_OK
    assert " ring ksplit2 fold(4 rows) masked" in lib.gemm_last_path(), lib.gemm_last_path()
    assert _v(lib, M=4101, N=1000, K=1032, tA=1, lda=4101) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith(
        "mfma t128x128x64 w2x2 a32x32x16 TN epi=beta0 ring masked staged"), lib.gemm_last_path()
    assert _v(lib, M=8193, N=1000, K=1032, tA=1, lda=8193) == lib.GEMM_OK
    assert "fold" not in lib.gemm_last_path(), lib.gemm_last_path()
    # (256 tiles, at most one per CU: with both operands straight into LDS
    # the deep ring, or the two-group form with ten half-slots when B is
    # N-contiguous and K at least 2048; with a staged operand K split over
    # two wave groups)
    assert _v(lib, M=4096, N=1000, K=1032, tA=1, lda=4104) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" TN epi=beta0 ring deep masked"), lib.gemm_last_path()
    assert _v(lib, M=4096, N=1000, K=2056, tA=1, lda=4104) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" TN epi=beta0 ring two-group deep masked"), \
        lib.gemm_last_path()
    assert _v(lib, M=4096, N=1000, K=1032, tA=1, tB=1, lda=4104) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" TT epi=beta0 ring deep masked"), lib.gemm_last_path()
    assert _v(lib, M=4096, N=1024, K=1028, tA=0, lda=1032) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" ring ksplit2 masked staged (A: K % 8 != 0)")
    assert _v(lib, M=4096, N=1000, K=1024, tA=0, tB=0, ldb=1000) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" NN epi=beta0 ring deep masked"), lib.gemm_last_path()
    assert _v(lib, M=4096, N=1004, K=1024, tA=0, tB=0, ldb=1008) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" ring ksplit2 masked staged (B: N % 8 != 0)")
    assert _v(lib, A=A0 + 2) == lib.GEMM_OK
    path = lib.gemm_last_path()
    assert path.startswith("mfma ") and "A: 2-byte loads, base address is not 16-byte aligned" in path
    assert _v(lib, A=A0 + 8) == lib.GEMM_OK
    assert "A: 8-byte loads, base address" in lib.gemm_last_path()
    assert _v(lib, ldb=72) == lib.GEMM_OK
    assert "narrow staging" not in lib.gemm_last_path()  # 144-byte pitch is fine
    assert _v(lib, ldb=67) == lib.GEMM_OK
    assert "narrow staging (B: 2-byte loads, row pitch 134 B" in lib.gemm_last_path()
    assert _v(lib, ldb=66) == lib.GEMM_OK
    assert "(B: 4-byte loads, row pitch 132 B" in lib.gemm_last_path()
    assert _v(lib, ldb=68) == lib.GEMM_OK
    assert "(B: 8-byte loads, row pitch 136 B" in lib.gemm_last_path()
    assert _v(lib, lda=67, ldb=67, M=64, N=64, K=64) == lib.GEMM_OK
    assert ("(A: 2-byte loads, row pitch 134 B is not a multiple of 16 B; "
            "B: 2-byte loads, row pitch 134 B") in lib.gemm_last_path()
    # whole 256x256 tiles with an unaligned operand: 128x128 tiles on the ring
    # kernel, B staged through registers
    assert _v(lib, M=8192, N=8192, K=8192, tB=1, dtype=1, ldb=8193) == lib.GEMM_OK
    assert lib.gemm_last_path() == ("mfma t128x128x64 w2x2 a32x32x16 NT epi=beta0 ring staged "
                                    "(B: row pitch 16386 B is not a multiple of 16 B)"), \
        lib.gemm_last_path()


def test_ring_modes(lib, monkeypatch):
    # at most one 128x128 tile per CU, both operands direct: the two-group
    # form with ten half-slots when B is N-contiguous and K >= 2048, else
    # the deep ring
    assert _v(lib, M=2048, N=2048, K=2048, dtype=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == \
        "mfma t128x128x64 w2x4 a32x32x16 NN epi=beta0 ring two-group deep"
    assert _v(lib, M=2048, N=2048, K=2048, dtype=1, tB=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == "mfma t128x128x64 w2x2 a32x32x16 NT epi=beta0 ring deep"
    # ... or two K groups when an operand is staged through registers
    assert _v(lib, M=2048, N=2048, K=2048, dtype=1, lda=2049) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith(
        "mfma t128x128x64 w2x2 a32x32x16 NN epi=beta0 ring ksplit2 staged (A: row pitch")
    # more tiles than CUs: two workgroups per CU, of two wave groups taking
    # turns (both operands direct) or of one group (a staged operand)
    assert _v(lib, M=4096, N=2048, K=1024, dtype=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == "mfma t128x128x64 w2x4 a32x32x16 NN epi=beta0 ring two-group"
    assert _v(lib, M=4096, N=2048, K=1024, dtype=1, lda=1025) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith(
        "mfma t128x128x64 w2x2 a32x32x16 NN epi=beta0 ring staged (A: row pitch")
    monkeypatch.setenv("GEMM_RING_MODE", "shared")
    assert _v(lib, M=2048, N=2048, K=2048, dtype=1) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" ring")
    monkeypatch.setenv("GEMM_RING_MODE", "ksplit2")
    assert _v(lib, M=4096, N=2048, K=1024, dtype=1) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" ring ksplit2")
    monkeypatch.setenv("GEMM_RING_MODE", "deep")
    assert _v(lib, M=4096, N=2048, K=1024, dtype=1) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" ring deep")
    assert _v(lib, M=2048, N=2048, K=2048, dtype=1, lda=2049) == lib.GEMM_ERR_UNSUPPORTED
    monkeypatch.setenv("GEMM_RING_MODE", "pp")
    assert _v(lib, M=4096, N=2048, K=1024, dtype=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == "mfma t128x128x64 w2x4 a32x32x16 NN epi=beta0 ring two-group"
    monkeypatch.setenv("GEMM_RING_MODE", "ppdeep")
    assert _v(lib, M=4096, N=2048, K=1024, dtype=1) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" ring two-group deep")
    assert _v(lib, M=2048, N=2048, K=2048, dtype=1, lda=2049) == lib.GEMM_ERR_UNSUPPORTED
    assert _v(lib, M=2048, N=2048, K=2048, dtype=1, lda=2049) == lib.GEMM_ERR_UNSUPPORTED
    monkeypatch.setenv("GEMM_RING_MODE", "wide")
    assert _v(lib, M=4096, N=2048, K=1024, dtype=1) == lib.GEMM_ERR_INVALID_ARG
    monkeypatch.delenv("GEMM_RING_MODE")
    monkeypatch.setenv("GEMM_STAGE_DEPTH", "1")
    assert _v(lib, M=2048, N=2048, K=2048, dtype=1, lda=2049) == lib.GEMM_OK
    monkeypatch.setenv("GEMM_STAGE_DEPTH", "3")
    assert _v(lib, M=2048, N=2048, K=2048, dtype=1, lda=2049) == lib.GEMM_ERR_INVALID_ARG


def test_ragged_dims_stay_on_mfma_masked(lib):
    assert _v(lib, M=4097, N=1000, K=1032, tA=1, lda=4104) == lib.GEMM_OK
    path = lib.gemm_last_path()
    assert path.startswith("mfma ") and " masked" in path, path
    assert _v(lib, M=16, N=8, K=16) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("mfma t16x16x64"), lib.gemm_last_path()


def test_k16_tail_is_named(lib):
    # 16x16x32 atoms (t16, t64): a last K step with 1..16 valid K-values
    assert _v(lib, M=16, N=8, K=16) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith("masked k16-tail"), lib.gemm_last_path()
    for K, tail in [(48, True), (40, True), (33, True), (56, False), (64, False), (1, True)]:
        assert _v(lib, M=200, N=200, K=K, lda=64, ldb=200) == lib.GEMM_OK
        assert ("k16-tail" in lib.gemm_last_path()) == tail, (K, lib.gemm_last_path())
    # 32x32x16 atoms have no tail form: their last K step multiplies the
    # staged zeros past K in every sub-step
    assert _v(lib, M=4096, N=4096, K=48, lda=64, ldb=4096) == lib.GEMM_OK
    assert "k16-tail" not in lib.gemm_last_path()


def test_f32_operand_dtypes(lib, monkeypatch):
    # 256x256 tiles in any layout: the two-group kernel rounds fragments as
    # it reads them (whole tiles: K a multiple of 32)
    assert _v(lib, M=8192, N=8192, K=8192, tB=1, dtype=lib.GEMM_DTYPE_F32_BF16) == lib.GEMM_OK
    assert lib.gemm_last_path() == "mfma t256x256x64 w2x4 a32x32x16 NT epi=beta0 pingpong f32->bf16"
    assert _v(lib, M=4096, N=4096, K=4096 + 32, tB=1, dtype=2, beta=1.0, C=D0) == lib.GEMM_OK
    assert lib.gemm_last_path() == "mfma t256x256x64 w2x4 a32x32x16 NT epi=acc+c pingpong f32->f16"
    for tA, tB, ops in ((0, 0, "NN"), (1, 0, "TN"), (1, 1, "TT")):
        assert _v(lib, M=4096, N=4096, K=4096, tA=tA, tB=tB, dtype=3) == lib.GEMM_OK
        assert lib.gemm_last_path() == \
            f"mfma t256x256x64 w2x4 a32x32x16 {ops} epi=beta0 pingpong f32->bf16"
    # edge tiles and K tails too, when every operand's contiguous dimension
    # is a multiple of 4 (whole 16-byte pieces)
    for kw in (dict(tB=0, M=8192 + 256 + 8), dict(tA=1, tB=1, N=8192 - 8),
               dict(tB=1, K=8192 + 16), dict(tA=1, tB=0, K=8192 + 3)):
        args = dict(M=8192, N=8192, K=8192, dtype=lib.GEMM_DTYPE_F32_BF16)
        args.update(kw)
        assert _v(lib, **args) == lib.GEMM_OK
        path = lib.gemm_last_path()
        assert path.startswith("mfma t256x256x64 w2x4 a32x32x16") and path.endswith(
            " pingpong masked f32->bf16"), (kw, path)
    # otherwise (a contiguous dimension cut inside a piece, rows not 16-byte
    # aligned) the 128x128 ring kernel stages both operands through registers
    # and rounds them there; edges or a K tail make it masked
    for kw in (dict(tA=1, M=8192 - 2), dict(tB=1, K=8192 + 2), dict(tB=1, lda=8192 + 2)):
        args = dict(M=8192, N=8192, K=8192, dtype=lib.GEMM_DTYPE_F32_BF16)
        args.update(kw)
        assert _v(lib, **args) == lib.GEMM_OK
        path = lib.gemm_last_path()
        masked = " masked" if ("K" in kw or "M" in kw or "N" in kw) else ""
        assert path.startswith("mfma t128x128x64 w2x2 a32x32x16") and path.endswith(
            f" ring{masked} f32->bf16 staged (A, B: float32 values rounded in registers)"), (kw, path)
    # large pitches (64-bit addressing) keep the masked general kernel
    assert _v(lib, M=256, N=256, K=256, tB=1, dtype=3, lda=1 << 22, A=1 << 40) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" masked f32->bf16"), lib.gemm_last_path()
    assert _v(lib, dtype=lib.GEMM_DTYPE_F32_F16) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith("masked f32->f16"), lib.gemm_last_path()
    # pitches count 4-byte elements: 66 floats = 264 B is 8-byte aligned only
    assert _v(lib, dtype=2, ldb=66) == lib.GEMM_OK
    assert "(B: 8-byte loads, row pitch 264 B" in lib.gemm_last_path(), lib.gemm_last_path()
    assert _v(lib, dtype=2, A=A0 + 4) == lib.GEMM_OK
    assert "(A: 4-byte loads, base address" in lib.gemm_last_path(), lib.gemm_last_path()
    assert _v(lib, dtype=2, A=A0 + 2) == lib.GEMM_ERR_INVALID_ARG  # floats must be 4-byte aligned
    # D must not overlap A's float32 extent (twice the 16-bit extent)
    assert _v(lib, dtype=0, M=64, K=64, D=A0 + 64 * 64 * 2 + 256) == lib.GEMM_OK
    assert _v(lib, dtype=2, M=64, K=64, D=A0 + 64 * 64 * 2 + 256) == lib.GEMM_ERR_ALIAS
    monkeypatch.setenv("GEMM_FORCE_PATH", "fma")
    assert _v(lib, dtype=3) == lib.GEMM_ERR_UNSUPPORTED


def _v8(lib, M=64, N=64, K=64, tA=0, tB=0, alpha=1, beta=0, A=A0, lda=None, B=B0, ldb=None,
        C=C0, ldc=None, D=D0, ldd=None):
    lda = lda if lda is not None else (M if tA else K)
    ldb = ldb if ldb is not None else (K if tB else N)
    ldc = ldc if ldc is not None else N
    ldd = ldd if ldd is not None else N
    return lib.gemm_i8_validate(M, N, K, tA, tB, alpha, beta, A, lda, B, ldb, C, ldc, D, ldd)


def test_fp8_dtypes_take_the_byte_kernel(lib, monkeypatch):
    assert _v(lib, dtype=lib.GEMM_DTYPE_F8_E4M3, tB=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == "fp8 e4m3 mfma t128x128x128 w2x2 a32x32x64 NT epi=beta0"
    assert _v(lib, dtype=lib.GEMM_DTYPE_F8_E5M2, tA=1, beta=0.5) == lib.GEMM_OK
    assert lib.gemm_last_path() == "fp8 e5m2 mfma t128x128x128 w2x2 a32x32x64 TN epi=general"
    assert _v(lib, dtype=4, A=A0 + 1, lda=65) == lib.GEMM_OK  # any alignment
    assert lib.gemm_last_path().endswith("bytewise staging")
    assert _v(lib, dtype=4, K=0, lda=1, A=0, B=0, beta=2.0) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("scale")
    # D must not overlap A's 64 x 64 bytes
    assert _v(lib, dtype=4, D=A0 + 64 * 64 - 4) == lib.GEMM_ERR_ALIAS
    assert _v(lib, dtype=4, D=A0 + 64 * 64) == lib.GEMM_OK
    monkeypatch.setenv("GEMM_FORCE_PATH", "fma")
    assert _v(lib, dtype=5) == lib.GEMM_ERR_UNSUPPORTED


def test_byte_two_group_kernel_cd_rows(lib):
    # whole 256x256 NT tiles take the two-group kernel on 16-wide atoms, whose
    # epilogue stores 16 bytes per lane when D (and C when read) have 16-byte
    # rows; otherwise the edge-tile form accesses C and D element by element
    assert _v8(lib, M=512, N=512, K=256, tB=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == "i8 mfma t256x256x128 w2x4 a16x16x64 NT epi=beta0 pingpong"
    assert _v(lib, M=512, N=512, K=256, tB=1, dtype=lib.GEMM_DTYPE_F8_E4M3) == lib.GEMM_OK
    assert lib.gemm_last_path() == "fp8 e4m3 mfma t256x256x128 w2x4 a16x16x128 NT epi=beta0 pingpong"
    assert _v8(lib, M=512, N=512, K=256, tB=1, ldd=514) == lib.GEMM_OK
    assert lib.gemm_last_path() == \
        "i8 mfma t256x256x128 w2x4 a16x16x64 NT epi=beta0 pingpong masked elementwise C/D"
    assert _v8(lib, M=512, N=512, K=256, tB=1, beta=1, C=D0, ldc=512) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" pingpong"), lib.gemm_last_path()
    assert _v8(lib, M=512, N=512, K=256, tB=1, beta=1, C=C0 + 4, ldc=512) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" pingpong masked elementwise C/D"), lib.gemm_last_path()
    # fewer than 4 tiles of 256x256: the 128x128 kernel
    assert _v8(lib, M=256, N=512, K=256, tB=1, ldd=514) == lib.GEMM_OK
    assert lib.gemm_last_path() == "i8 mfma t128x128x128 w2x2 a32x32x32 NT epi=beta0"


def test_byte_two_group_kernel_edge_tiles(lib):
    # other shapes take the two-group kernel with edge tiles when K is a
    # multiple of 16, an M/N-contiguous operand's contiguous dimension of 16,
    # and the grid has at least 4 tiles of 256x256 (C and D element by
    # element when N % 4 != 0)
    assert _v8(lib, M=1000, N=1000, K=1024, tB=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == "i8 mfma t256x256x128 w2x4 a16x16x64 NT epi=beta0 pingpong masked"
    assert _v(lib, M=1008, N=1008, K=1040, dtype=lib.GEMM_DTYPE_F8_E5M2) == lib.GEMM_OK
    assert lib.gemm_last_path() == \
        "fp8 e5m2 mfma t256x256x128 w2x4 a16x16x128 NN epi=beta0 pingpong masked"
    for kw in (dict(K=1000, tB=1),            # K % 16 != 0
               dict(N=1000),                  # B stored [K][N], N % 16 != 0
               dict(M=1000, tA=1, tB=1),      # A stored [K][M], M % 16 != 0
               dict(M=500, N=200, tB=1)):     # 2 tiles of 256x256
        args = dict(M=1008, N=1008, K=1024)
        args.update(kw)
        assert _v8(lib, **args) == lib.GEMM_OK
        assert lib.gemm_last_path().startswith("i8 mfma t128x128x128"), (kw, lib.gemm_last_path())


def test_byte_two_group_kernel_elementwise_cd(lib):
    assert _v8(lib, M=1008, N=1002, K=1024, tB=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == \
        "i8 mfma t256x256x128 w2x4 a16x16x64 NT epi=beta0 pingpong masked elementwise C/D"
    assert _v(lib, M=4097, N=4097, K=4096, tB=1, dtype=lib.GEMM_DTYPE_F8_E5M2) == lib.GEMM_OK
    assert lib.gemm_last_path() == ("fp8 e5m2 mfma t256x256x128 w2x4 a16x16x128 NT epi=beta0 "
                                    "pingpong masked elementwise C/D")


def test_i8_form_checks_and_paths(lib):
    assert _v8(lib, tB=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == "i8 mfma t128x128x128 w2x2 a32x32x32 NT epi=beta0"
    assert _v8(lib, beta=-2, tA=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == "i8 mfma t128x128x128 w2x2 a32x32x32 TN epi=general"
    assert _v8(lib, lda=65) == lib.GEMM_OK  # any alignment: bytewise staging
    assert lib.gemm_last_path().endswith("bytewise staging")
    assert _v8(lib, A=A0 + 1) == lib.GEMM_OK
    assert _v8(lib, K=0, A=0, B=0, beta=3, lda=1) == lib.GEMM_OK
    assert "D = beta*C" in lib.gemm_last_path()
    assert _v8(lib, alpha=0, A=0, B=0, beta=0) == lib.GEMM_OK
    assert _v8(lib, M=0, A=0, B=0, D=0) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("noop")
    assert _v8(lib, M=-1) == lib.GEMM_ERR_INVALID_ARG
    assert _v8(lib, lda=63) == lib.GEMM_ERR_INVALID_ARG
    assert _v8(lib, D=0) == lib.GEMM_ERR_INVALID_ARG
    assert _v8(lib, D=D0 + 2) == lib.GEMM_ERR_INVALID_ARG
    assert _v8(lib, beta=1, C=0) == lib.GEMM_ERR_INVALID_ARG
    assert _v8(lib, A=0) == lib.GEMM_ERR_INVALID_ARG
    assert _v8(lib, beta=1, C=D0) == lib.GEMM_OK  # exact in-place
    assert _v8(lib, beta=1, C=D0 + 4) == lib.GEMM_ERR_ALIAS
    assert _v8(lib, D=A0 + 64) == lib.GEMM_ERR_ALIAS
    # A is 64 x 64 bytes: a D placed right after it does not overlap
    assert _v8(lib, D=A0 + 64 * 64) == lib.GEMM_OK
    assert _v8(lib, M=1 << 31) == lib.GEMM_ERR_UNSUPPORTED


def test_huge_pitch_takes_64bit_addressing(lib):
    # 64 rows (the 64x64 tile) of a 16M-element pitch overflow 32-bit offsets
    assert _v(lib, M=256, N=256, K=256, lda=1 << 24, A=1 << 40) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith("masked"), lib.gemm_last_path()
    assert _v(lib, M=256, N=256, K=256, lda=1 << 20) == lib.GEMM_OK
    assert not lib.gemm_last_path().endswith("masked")


def test_tile_and_epilogue_choice(lib):
    assert _v(lib, M=8192, N=8192, K=8192, tB=1, dtype=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == "mfma t256x256x64 w2x4 a16x16x32 NT epi=beta0 pingpong"
    assert _v(lib, M=4096, N=4096, K=4096, dtype=1, beta=1.0, C=D0) == lib.GEMM_OK
    assert lib.gemm_last_path() == "mfma t256x256x64 w2x4 a16x16x32 NN epi=acc+c pingpong"
    # A stored [K][M]: the two-group kernel keeps the 32x32x16 atom
    assert _v(lib, M=4096, N=4096, K=4096, tA=1, dtype=1) == lib.GEMM_OK
    assert lib.gemm_last_path() == "mfma t256x256x64 w2x4 a32x32x16 TN epi=beta0 pingpong"
    # fewer 256x256 tiles than CUs: that tile still, once K is long enough
    for M, N, K, tile in [(3072, 4096, 1024, 256), (3072, 4096, 512, 128),
                          (1024, 8192, 2048, 256), (4096, 2048, 1024, 128),
                          (2048, 2048, 8192, 128)]:
        assert _v(lib, M=M, N=N, K=K, tB=1, dtype=1) == lib.GEMM_OK
        assert lib.gemm_last_path().startswith(f"mfma t{tile}x{tile}x64"), \
            (M, N, K, lib.gemm_last_path())
    assert _v(lib, M=512, N=512, K=512, alpha=1.5, beta=0.5) == lib.GEMM_OK
    assert lib.gemm_last_path() == "mfma t32x32x64k4 w1x1 a32x32x16 NN epi=general ksplit4"


def test_two_group_kernel_edge_tiles(lib, monkeypatch):
    # 256x256 tiles that need masking stay on the two-group kernel when the
    # operands load in whole 16-byte pieces and the grid fills its last round
    # of 256 CUs to at least 3/4
    assert _v(lib, M=4000, N=4000, K=4096, tB=1, dtype=1) == lib.GEMM_OK  # 256 tiles
    assert lib.gemm_last_path() == "mfma t256x256x64 w2x4 a16x16x32 NT epi=beta0 pingpong masked"
    assert _v(lib, M=8000, N=8000, K=8200, beta=1.0, C=D0) == lib.GEMM_OK  # 1024 tiles
    assert lib.gemm_last_path() == "mfma t256x256x64 w2x4 a16x16x32 NN epi=acc+c pingpong masked"
    assert _v(lib, M=4000, N=3904, K=4100, tA=1) == lib.GEMM_OK  # K tail: both M/N-contiguous
    assert lib.gemm_last_path() == "mfma t256x256x64 w2x4 a32x32x16 TN epi=beta0 pingpong masked"
    for kw in (dict(M=4353, N=4353),           # 324 tiles: the second round 27 % full
               dict(K=4100),                   # K-contiguous operand, K % 8 != 0
               dict(M=4004, tA=1),             # A stored [K][M], M % 8 != 0
               dict(N=4004, tB=0),             # B stored [K][N], N % 8 != 0
               dict(A=A0 + 2),                 # A not 16-byte aligned
               dict(dtype=2, K=4098)):         # float32 operands, K % 4 != 0
        args = dict(M=4000, N=4000, K=4096, tB=1)
        args.update(kw)
        assert _v(lib, **args) == lib.GEMM_OK
        assert lib.gemm_last_path().startswith("mfma t128x128x64"), (kw, lib.gemm_last_path())
    # float32 operands: the contiguous dimensions in multiples of 4
    assert _v(lib, M=4000, N=4000, K=4100, tB=1, dtype=2) == lib.GEMM_OK
    assert lib.gemm_last_path() == \
        "mfma t256x256x64 w2x4 a32x32x16 NT epi=beta0 pingpong masked f32->f16"
    # a forced 256x256 tile skips the fill test
    monkeypatch.setenv("GEMM_FORCE_TILE", "t256x256x64")
    assert _v(lib, M=4097, N=4097, K=4096, tB=1) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" pingpong masked"), lib.gemm_last_path()
    assert _v(lib, M=96, N=40, K=20, tA=1, tB=0) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" pingpong masked"), lib.gemm_last_path()


def test_split_past_a_multiple_of_the_tile(lib, monkeypatch):
    # at most 128 rows and columns past the last whole 256x256 tile that add a
    # round of tiles: whole tiles, remainder rows, remainder columns, each
    # planned on its own and launched in that order
    assert _v(lib, M=4097, N=4097, K=4096, tB=1, dtype=1) == lib.GEMM_OK
    path = lib.gemm_last_path()
    assert path.startswith("split core 4096x4096: mfma t256x256x64 w2x4 a16x16x32 NT epi=beta0 "
                           "pingpong; rows 1x4097: mfma ") and "; cols 4096x1: mfma " in path, path
    assert _v(lib, M=4128, N=8192, K=1024, tA=1, dtype=0, beta=1.0, C=D0) == lib.GEMM_OK
    path = lib.gemm_last_path()
    assert path.startswith("split core 4096x8192: mfma t256x256x64 w2x4 a32x32x16 TN epi=acc+c "
                           "pingpong; rows 32x8192: mfma ") and "cols" not in path, path
    assert _v(lib, M=4096, N=4100, K=512, tB=1, dtype=3) == lib.GEMM_OK
    path = lib.gemm_last_path()
    assert path.startswith("split core 4096x4096: mfma t256x256x64 w2x4 a32x32x16 NT epi=beta0 "
                           "pingpong f32->bf16; cols 4096x4: mfma ") and "rows" not in path, path
    for kw in (dict(M=4353, N=4353),           # the remainder adds no round
               dict(M=4096 + 129),             # more than 128 remainder rows
               dict(N=4097, tB=0),             # B [K][N] with an unaligned row pitch
               dict(N=4097, K=0, beta=1.0, lda=1, ldb=1),  # D = beta*C
               dict(M=3841, N=4097)):          # fewer than 256 whole tiles
        args = dict(M=4097, N=4096, K=4096, tB=1, dtype=1)
        args.update(kw)
        assert _v(lib, **args) == lib.GEMM_OK
        assert not lib.gemm_last_path().startswith("split"), (kw, lib.gemm_last_path())
    monkeypatch.setenv("GEMM_FORCE_TILE", "t256x256x64")
    assert _v(lib, M=4097, N=4097, K=4096, tB=1, dtype=1) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith(" pingpong masked"), lib.gemm_last_path()


def test_k_split_eight_ways(lib):
    # one round of 32x32 tiles and K >= 2048: K split over eight one-wave groups
    for M, N, K in [(1, 4097, 4096), (4096, 1, 4096), (256, 1024, 4096)]:
        assert _v(lib, M=M, N=N, K=K, tB=1, dtype=1) == lib.GEMM_OK
        assert lib.gemm_last_path().startswith("mfma t32x32x64k8 w1x1 a32x32x16 NT"), \
            (M, N, K, lib.gemm_last_path())
        assert " ksplit8" in lib.gemm_last_path()
    # more than one round, or a shorter K: four groups
    for M, N, K in [(1, 8193, 8192), (64, 4160, 4096), (512, 512, 512), (256, 1024, 1024)]:
        assert _v(lib, M=M, N=N, K=K, tB=1, dtype=1) == lib.GEMM_OK
        assert lib.gemm_last_path().startswith("mfma t32x32x64k4 "), (M, N, K, lib.gemm_last_path())


def test_k_split_tile_choice(lib):
    # 64x64 tiles would leave CUs idle: 32x32 tiles, K split over 4 wave groups
    assert _v(lib, M=1000, N=500, K=256) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("mfma t32x32x64k4 ")
    assert " ksplit4 masked" in lib.gemm_last_path()
    # too little K for four groups of 64
    assert _v(lib, M=512, N=512, K=255) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("mfma t64x64x64 ")
    # 256 tiles of 64x64 fill the chip: with K >= 2048 and whole tiles, K is
    # split over four groups of 2x2 waves; with edges, 64x64 tiles (K < 4096)
    # or 32x32 tiles in four K groups (K >= 4096); with a short K, 64x64
    assert _v(lib, M=1024, N=1024, K=2048) == lib.GEMM_OK
    assert lib.gemm_last_path() == "mfma t64x64x64k4 w2x2 a16x16x32 NN epi=beta0 ksplit4"
    assert _v(lib, M=128, N=8192, K=8192, tB=1) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("mfma t64x64x64k4 "), lib.gemm_last_path()
    assert _v(lib, M=1000, N=1024, K=2048) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("mfma t64x64x64 "), lib.gemm_last_path()
    assert _v(lib, M=1000, N=1024, K=4096) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("mfma t32x32x64k4 "), lib.gemm_last_path()
    assert _v(lib, M=1024, N=1024, K=1024) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("mfma t64x64x64 "), lib.gemm_last_path()
    # whole tiles, but K not a multiple of 4 x 64: the groups' last steps are masked
    assert _v(lib, M=512, N=512, K=512 + 64) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith("ksplit4 masked"), lib.gemm_last_path()
    assert _v(lib, M=512, N=512, K=1024) == lib.GEMM_OK
    assert lib.gemm_last_path().endswith("ksplit4"), lib.gemm_last_path()


def test_force_path_and_tile(lib, monkeypatch):
    monkeypatch.setenv("GEMM_FORCE_PATH", "fma")
    assert _v(lib) == lib.GEMM_OK
    assert "forced by GEMM_FORCE_PATH=fma" in lib.gemm_last_path()
    monkeypatch.setenv("GEMM_FORCE_PATH", "mfma")
    assert _v(lib, A=A0 + 2) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("mfma "), lib.gemm_last_path()
    monkeypatch.setenv("GEMM_FORCE_PATH", "bogus")
    assert _v(lib) == lib.GEMM_ERR_INVALID_ARG
    monkeypatch.delenv("GEMM_FORCE_PATH")
    monkeypatch.setenv("GEMM_FORCE_TILE", "t128x128x64")
    assert _v(lib, M=8192, N=8192, K=8192) == lib.GEMM_OK
    assert lib.gemm_last_path().startswith("mfma t128x128x64")
    monkeypatch.setenv("GEMM_FORCE_TILE", "t7x7")
    assert _v(lib) == lib.GEMM_ERR_INVALID_ARG


def test_debug_log_names_the_path_and_its_reason():
    code = (
        "import dense_gemm_tile_amd as d\n"
        "d.gemm_validate(4097,1000,1032,0,1,0,2.0,-1.0,0x10000000,4097,0x20000000,1000,"
        "0x30000000,1000,0x40000000,1000)\n"
        "d.gemm_validate(-1,1,1,0,0,0,1.0,0.0,0,1,0,1,0,1,0,1)\n")
    env = dict(os.environ, GEMM_LOG="debug", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("[gemm]")]
    assert len(lines) == 2
    assert "M=4097 N=1000 K=1032 -> mfma " in lines[0] and "row pitch 8194 B" in lines[0]
    assert "error 1: negative dimension" in lines[1]


@pytest.mark.parametrize("tiles_m,tiles_n,group", [
    (1, 1, 8), (32, 32, 8), (16, 16, 8), (17, 4, 8), (33, 8, 8), (65, 16, 8), (3, 100, 8),
    (100, 3, 4), (7, 9, 1), (8, 8, 16), (257, 1, 8), (1, 257, 8)])
def test_tile_order_is_a_bijection(lib, tiles_m, tiles_n, group):
    tm, tn = lib.gemm_tile_order(tiles_m, tiles_n, group)
    pairs = set(zip(tm, tn))
    assert len(pairs) == tiles_m * tiles_n
    assert all(0 <= m < tiles_m and 0 <= n < tiles_n for m, n in pairs)


def test_tile_order_keeps_an_xcd_on_a_compact_block(lib):
    # 32 x 32 tiles: the first 32 workgroups each XCD runs (ids x, x+8, ...)
    # should cover few row and column panels (8 rows x 4 columns in grouped order).
    tm, tn = lib.gemm_tile_order(32, 32, 8)
    for xcd in range(8):
        ids = [xcd + 8 * i for i in range(32)]
        rows = {tm[w] for w in ids}
        cols = {tn[w] for w in ids}
        assert len(rows) * len(cols) <= 32, (xcd, len(rows), len(cols))


def test_tile_order_rejects_bad_arguments(lib):
    with pytest.raises(lib.GemmError):
        lib.gemm_tile_order(0, 4, 8)
    with pytest.raises(lib.GemmError):
        lib.gemm_tile_order(4, 4, 0)
