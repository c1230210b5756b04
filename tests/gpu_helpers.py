"""Helpers shared by the GPU tests: upload seeded inputs, call the library
through its C ABI on the current torch stream, and judge the result against
the CPU oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

NAN16 = {"f16": 0x7E00, "bf16": 0x7FC0}
D_SENTINEL = 0x7FC0DEAD  # a NaN bit pattern no kernel ever writes


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import dense_gemm_tile_amd  # noqa: F401  (fails loudly if the library is not built)


def say(msg: str):
    """Name the case on stderr before its GPU work starts."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def poison_padding(x: torch.Tensor, cols: int, dtype: str) -> torch.Tensor:
    """Fill the columns past `cols` of a padded [rows, ld] operand with NaNs."""
    x = x.clone()
    if x.shape[1] > cols:
        if x.dtype == torch.float32:
            x[:, cols:] = float("nan")
        else:
            x.view(torch.int16)[:, cols:] = int(np.uint16(NAN16[dtype]).view(np.int16))
    return x


class Run:
    """One call's inputs (host copies) and its device result."""

    def __init__(self, cfg: workloads.Config, inp: workloads.Inputs, D: torch.Tensor, path: str):
        self.cfg, self.inp, self.D, self.path = cfg, inp, D, path

    def oracle_args(self):
        c = self.cfg
        lda, ldb, ldc, _ = c.lds()
        A = workloads.bits_u16(self.inp.A).reshape(-1)
        B = workloads.bits_u16(self.inp.B).reshape(-1)
        C = self.inp.C.numpy().reshape(-1) if self.inp.C is not None else None
        dt = workloads.DTYPE_CODE[c.dtype]
        return (c.M, c.N, c.K, dt, c.transA, c.transB, c.alpha, c.beta, A, lda, B, ldb, C, ldc)

    def reference(self, rows=None):
        c = self.cfg
        if c.dtype.startswith("f32_"):
            # float32 operands: the oracle rounds them itself (f16 or bf16)
            lda, ldb, ldc, _ = c.lds()
            dt = 0 if c.dtype == "f32_f16" else 1
            C = self.inp.C.numpy().reshape(-1) if self.inp.C is not None else None
            return oracle.gemm_reference_f32(
                c.M, c.N, c.K, dt, c.transA, c.transB, c.alpha, c.beta,
                self.inp.A.numpy().reshape(-1), lda, self.inp.B.numpy().reshape(-1), ldb,
                C, ldc, rows=rows)
        return oracle.gemm_reference(*self.oracle_args(), rows=rows)

    def check(self, rows=None):
        """Elementwise oracle check (on `rows` if given); returns the report."""
        D_ref, bound = self.reference(rows)
        got = self.D[:, : self.cfg.N].numpy().astype(np.float64)
        if rows is not None:
            got = got[rows]
        rep = oracle.check(got, D_ref, bound)
        assert rep["ok"], (self.cfg, self.path, rep)
        return rep

    def check_elements(self, block: int = 64, seed: int = 0):
        """One element at a random position inside every block x block region
        of D, each against its own dot product in the oracle."""
        c = self.cfg
        rng = np.random.default_rng(seed)
        I, J = [], []
        for i0 in range(0, c.M, block):
            for j0 in range(0, c.N, block):
                I.append(rng.integers(i0, min(c.M, i0 + block)))
                J.append(rng.integers(j0, min(c.N, j0 + block)))
        I, J = np.array(I, dtype=np.int64), np.array(J, dtype=np.int64)
        D_ref, bound = oracle.gemm_reference_elements(*self.oracle_args(), I, J)
        got = self.D.numpy()[I, J].astype(np.float64)
        rep = oracle.check(got, D_ref, bound)
        assert rep["ok"], (self.cfg, self.path, rep)
        return rep

    def check_padding_untouched(self):
        _, _, _, ldd = self.cfg.lds()
        if ldd > self.cfg.N and not self.cfg.inplace:
            pad = self.D[:, self.cfg.N:].contiguous().view(torch.int32).numpy().view(np.uint32)
            assert np.all(pad == D_SENTINEL), "kernel wrote past column N"


def _shifted(x: torch.Tensor, dev, off: int) -> torch.Tensor:
    """x on the device, starting `off` elements past an allocation's start
    (off = 1 gives a base address 2 bytes past a 16-byte boundary)."""
    if off == 0:
        return x.to(dev)
    flat = torch.zeros(off + x.numel(), dtype=x.dtype)
    flat[off:] = x.reshape(-1)
    return flat.to(dev)[off:].view(x.shape)


def run(cfg: workloads.Config, inp: workloads.Inputs | None = None, *, poison=True,
        stream=None, D_init=None, a_off=0, b_off=0) -> Run:
    import dense_gemm_tile_amd as dgt
    if inp is None:
        inp = workloads.make_inputs(cfg)
    lda, ldb, ldc, ldd = cfg.lds()
    a_cols = cfg.M if cfg.transA else cfg.K
    b_cols = cfg.K if cfg.transB else cfg.N
    A_h = poison_padding(inp.A, a_cols, cfg.dtype) if poison else inp.A
    B_h = poison_padding(inp.B, b_cols, cfg.dtype) if poison else inp.B
    inp = workloads.Inputs(cfg, inp.A_src, inp.B_src, A_h, B_h, inp.C)
    dev = torch.device("cuda:0")
    A = _shifted(A_h, dev, a_off)
    B = _shifted(B_h, dev, b_off)
    if cfg.inplace:
        assert inp.C is not None and ldc == ldd
        D = inp.C.to(dev).clone()
        C = D
    else:
        C = inp.C.to(dev) if inp.C is not None else None
        if D_init is not None:
            D = D_init.to(dev).clone()
        else:
            D = torch.empty((max(cfg.M, 1), ldd), dtype=torch.float32, device=dev)
            D.view(torch.int32).fill_(int(np.uint32(D_SENTINEL).view(np.int32)))
    say(f"{cfg.name} M={cfg.M} N={cfg.N} K={cfg.K} {cfg.dtype} tA={cfg.transA} "
        f"tB={cfg.transB} a={cfg.alpha} b={cfg.beta} lds={cfg.lds()} "
        f"offs={a_off},{b_off} "
        f"force={os.environ.get('GEMM_FORCE_PATH')}/{os.environ.get('GEMM_FORCE_TILE')}")
    s = stream if stream is not None else torch.cuda.current_stream()
    dgt.gemm(cfg.M, cfg.N, cfg.K, cfg.dtype, cfg.transA, cfg.transB, cfg.alpha, cfg.beta,
             A, lda, B, ldb, C, ldc, D, ldd, stream=s)
    path = dgt.gemm_last_path()
    torch.cuda.synchronize()
    return Run(cfg, inp, D.cpu(), path)


def sample_rows(M: int, tile: int = 256, per_tile: int = 2, seed: int = 0) -> np.ndarray:
    """Rows that touch every tile row band: its first and last rows plus random ones."""
    rng = np.random.default_rng(seed)
    rows = set()
    for t0 in range(0, M, tile):
        t1 = min(M, t0 + tile)
        rows.update({t0, t1 - 1})
        rows.update(rng.integers(t0, t1, per_tile).tolist())
    return np.array(sorted(rows), dtype=np.int64)
