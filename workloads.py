"""Seeded synthetic inputs for the dense GEMM D = alpha*op(A)@op(B) + beta*C.

This module only draws random numbers and packs them into the storage layout a
caller hands to a GEMM. It holds none of the contraction's arithmetic, so both
the CPU oracle (tests) and the HIP path (tests, bench) may take their inputs
from it without sharing any of the method's code.

Storage convention (row-major everywhere, following the TIRx gemm page's
"Algorithm" step 1, which normalises A to [M,K] and B to [K,N] and treats the
transpose flags as the stored orientation):
  transA=0 -> A stored [M,K], lda >= K;   transA=1 -> A stored [K,M], lda >= M
  transB=0 -> B stored [K,N], ldb >= N;   transB=1 -> B stored [N,K], ldb >= K
  C, D stored [M,N] in float32 with ldc, ldd >= N.

Distributions: "uniform[-1,1]" is torch.rand*2-1 in float32; "normal(0,s)" is
torch.randn*s with s the standard deviation. Half-precision operands are made
by drawing float32 and rounding with torch (round-to-nearest-even). C is never
rounded.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

# "f32_f16" / "f32_bf16": A and B are handed over as float32 and rounded to
# f16 / bf16 by the library while it stages them.
DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32_f16": torch.float32,
          "f32_bf16": torch.float32}
DTYPE_CODE = {"f16": 0, "bf16": 1, "f32_f16": 2, "f32_bf16": 3}


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    M: int
    N: int
    K: int
    dtype: str            # "f16" | "bf16"
    transA: int
    transB: int
    alpha: float
    beta: float
    dist: str             # "uniform" | "normal" | "normal_invsqrtk"
    seed: int
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    ldd: Optional[int] = None
    inplace: bool = False  # D aliases C (same buffer, ldc == ldd)

    def lds(self):
        lda = self.lda if self.lda is not None else (self.M if self.transA else self.K)
        ldb = self.ldb if self.ldb is not None else (self.K if self.transB else self.N)
        ldc = self.ldc if self.ldc is not None else self.N
        ldd = self.ldd if self.ldd is not None else self.N
        return lda, ldb, ldc, ldd

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The five workloads: a single 16x8x16 atom, a general-epilogue 512^3 case,
# the in-place accumulate 4096^3 case, the compute-bound 8192^3 NT case and a
# ragged transposed-A case whose A rows are not 16-byte aligned.
CONFIGS = {
    "atom16x8x16": Config("atom16x8x16", 16, 8, 16, "f16", 0, 0, 1.0, 0.0, "uniform", 1001),
    "gemm512": Config("gemm512", 512, 512, 512, "f16", 0, 0, 1.5, 0.5, "uniform", 1002),
    "gemm4096_inplace": Config("gemm4096_inplace", 4096, 4096, 4096, "bf16", 0, 0, 1.0, 1.0,
                               "normal", 1003, inplace=True),
    "gemm8192_nt": Config("gemm8192_nt", 8192, 8192, 8192, "bf16", 0, 1, 1.0, 0.0,
                          "normal_invsqrtk", 1004),
    "ragged4097x1000x1032_tn": Config("ragged4097x1000x1032_tn", 4097, 1000, 1032, "f16", 1, 0,
                                      2.0, -1.0, "uniform", 1005),
}
CONFIG_ORDER = ["atom16x8x16", "gemm512", "gemm4096_inplace", "gemm8192_nt",
                "ragged4097x1000x1032_tn"]

# Extra measurement case (not one of the five): float32 operands rounded to
# bf16 while staged, the 4096^3 NT shape with normal(0, 1/sqrt(K)) inputs.
EXTRA_CONFIGS = {
    "gemm4096_f32in_nt": Config("gemm4096_f32in_nt", 4096, 4096, 4096, "f32_bf16", 0, 1, 1.0,
                                0.0, "normal_invsqrtk", 1006),
}


def _draw(gen: torch.Generator, shape, dist: str, K: int) -> torch.Tensor:
    if dist == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    if dist == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32)
    if dist == "normal_invsqrtk":
        return torch.randn(shape, generator=gen, dtype=torch.float32) * (1.0 / math.sqrt(K))
    raise ValueError(dist)


def _pad_rows(x: torch.Tensor, ld: int) -> torch.Tensor:
    """Return a [rows, ld] buffer whose first x.shape[1] columns hold x."""
    rows, cols = x.shape
    if ld == cols:
        return x.contiguous()
    out = torch.zeros((rows, ld), dtype=x.dtype)
    out[:, :cols] = x
    return out


@dataclasses.dataclass
class Inputs:
    """Host (CPU) tensors in storage layout, plus the float32 sources."""
    cfg: Config
    A_src: torch.Tensor        # float32, stored shape, before rounding
    B_src: torch.Tensor
    A: torch.Tensor            # f16/bf16, stored shape [rows, ld]
    B: torch.Tensor
    C: Optional[torch.Tensor]  # float32 [M, ldc] or None when beta == 0


def make_inputs(cfg: Config, *, A_src: Optional[torch.Tensor] = None,
                B_src: Optional[torch.Tensor] = None, C: Optional[torch.Tensor] = None,
                want_c: Optional[bool] = None) -> Inputs:
    """Draw A, then B, then C (float32, CPU, seeded) in their stored shapes.

    Callers may pass explicit float32 sources (structured cases such as
    identity or integer-valued matrices); those are rounded the same way.
    """
    gen = torch.Generator("cpu").manual_seed(cfg.seed)
    lda, ldb, ldc, _ = cfg.lds()
    a_shape = (cfg.K, cfg.M) if cfg.transA else (cfg.M, cfg.K)
    b_shape = (cfg.N, cfg.K) if cfg.transB else (cfg.K, cfg.N)
    if A_src is None:
        A_src = _draw(gen, a_shape, cfg.dist, cfg.K)
    if B_src is None:
        B_src = _draw(gen, b_shape, cfg.dist, cfg.K)
    if want_c is None:
        want_c = cfg.beta != 0.0
    if C is None and want_c:
        C = _draw(gen, (cfg.M, cfg.N), cfg.dist if cfg.dist != "normal_invsqrtk" else "normal",
                  cfg.K)
    A_src = _pad_rows(A_src.float(), lda)
    B_src = _pad_rows(B_src.float(), ldb)
    tdt = DTYPES[cfg.dtype]
    A = A_src.to(tdt)
    B = B_src.to(tdt)
    if C is not None:
        C = _pad_rows(C.float(), ldc)
    return Inputs(cfg, A_src, B_src, A, B, C)


def bits_u16(x: torch.Tensor):
    """The raw 16-bit patterns of an f16/bf16 CPU tensor, as a numpy uint16 array."""
    return x.contiguous().view(torch.int16).numpy().view("uint16")


def with_shape(cfg: Config, **kw) -> Config:
    return dataclasses.replace(cfg, **kw)


def make_i8_inputs(M: int, N: int, K: int, transA: int, transB: int, seed: int):
    """Seeded int8 operands, uniform over [-128, 127], in their stored shapes
    (A then B, packed leading dimensions)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    a_shape = (K, M) if transA else (M, K)
    b_shape = (N, K) if transB else (K, N)
    A = torch.randint(-128, 128, a_shape, generator=gen, dtype=torch.int8)
    B = torch.randint(-128, 128, b_shape, generator=gen, dtype=torch.int8)
    return A, B


def fp8_finite_codes(fmt: int) -> torch.Tensor:
    """The 8-bit codes of finite values: E4M3 (fmt 4) excludes its two NaN
    codes S.1111.111, E5M2 (fmt 5) its exponent-31 codes (infinities, NaNs)."""
    c = torch.arange(256, dtype=torch.int32)
    if fmt == 4:
        keep = (c & 0x7F) != 0x7F
    else:
        keep = ((c >> 2) & 0x1F) != 0x1F
    return c[keep].to(torch.uint8)


def make_fp8_inputs(M: int, N: int, K: int, transA: int, transB: int, fmt: int, seed: int,
                    lda: Optional[int] = None, ldb: Optional[int] = None):
    """Seeded 8-bit float operands: codes drawn uniformly from the format's
    finite codes, in their stored shapes [rows, ld] (A then B)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    codes = fp8_finite_codes(fmt)
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    lda = lda or a_cols
    ldb = ldb or b_cols
    A = codes[torch.randint(0, codes.numel(), (a_rows, lda), generator=gen)]
    B = codes[torch.randint(0, codes.numel(), (b_rows, ldb), generator=gen)]
    return A, B

