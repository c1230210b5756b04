"""Stream capture: gemm() enqueues kernel launches only (no allocation, no
memset, no synchronisation), so calls captured into a HIP graph replay to the
same D as the eager calls, bit for bit, replay after replay, with eager work
on the same buffers between the replays. One case per kernel family that
the planner picks on its own, including C == D (reset before each replay)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import need_gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    # (M, N, K, dtype, tA, tB, alpha, beta, lda, in place, expected path prefix)
    (512, 512, 512, "f16", 0, 0, 1.5, 0.5, None, False, "mfma t32x32x64k4"),
    (4097, 1000, 1032, "f16", 1, 0, 2.0, -1.0, 4097, False, "mfma t128x128x64"),
    (2048, 2048, 2048, "bf16", 0, 1, 1.0, 0.0, None, False, "mfma t128x128x64"),
    (4096, 4096, 512, "bf16", 0, 0, 1.0, 1.0, None, True, "mfma t256x256x64"),
    (4000, 4000, 1032, "bf16", 1, 1, 1.0, 0.0, None, False, "mfma t256x256x64"),
    (3072, 4096, 1024, "f32_bf16", 0, 1, 1.0, 0.0, None, False, "mfma t256x256x64"),
    (1024, 1024, 1024, "f8e4m3", 0, 1, 1.0, 0.5, None, False, "fp8 e4m3 mfma"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}_{c[3]}")
def test_captured_calls_replay_bitwise(case, monkeypatch):
    need_gpu()
    import dense_gemm_tile_amd as dgt
    monkeypatch.delenv("GEMM_FORCE_PATH", raising=False)
    monkeypatch.delenv("GEMM_FORCE_TILE", raising=False)
    monkeypatch.delenv("GEMM_RING_MODE", raising=False)
    M, N, K, dtype, tA, tB, alpha, beta, lda, inplace, prefix = case
    dev = torch.device("cuda:0")
    if dtype == "f8e4m3":
        # finite E4M3 codes, drawn like the other operands: seeded, on the CPU
        gen = torch.Generator("cpu").manual_seed(801)
        codes = workloads.fp8_finite_codes(4)
        A = codes[torch.randint(0, len(codes), (M, K), generator=gen)].to(torch.uint8).to(dev)
        B = codes[torch.randint(0, len(codes), (N, K), generator=gen)].to(torch.uint8).to(dev)
        C0 = (torch.rand((M, N), generator=gen) * 2 - 1).to(dev)
        lda, ldb, ldc, ldd = K, K, N, N
    else:
        cfg = workloads.Config(f"graph{M}x{N}x{K}", M, N, K, dtype, tA, tB, alpha, beta,
                               "uniform", 800 + M % 97, lda=lda, inplace=inplace)
        inp = workloads.make_inputs(cfg)
        lda, ldb, ldc, ldd = cfg.lds()
        A, B = inp.A.to(dev), inp.B.to(dev)
        C0 = inp.C.to(dev) if inp.C is not None else None
    D = torch.empty((M, ldd), dtype=torch.float32, device=dev)
    say(f"graph case {case}")

    def call(stream):
        C = D if inplace else C0
        dgt.gemm(M, N, K, dtype, tA, tB, alpha, beta, A, lda, B, ldb, C, ldc, D, ldd,
                 stream=stream)

    def reset():
        if inplace:
            D.copy_(C0)
        else:
            D.fill_(float("nan"))

    reset()
    call(torch.cuda.current_stream())
    assert dgt.gemm_last_path().startswith(prefix), dgt.gemm_last_path()
    torch.cuda.synchronize()
    eager = D.clone()
    assert torch.isfinite(eager[:, :N]).all()

    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        reset()  # eager work on the graph's buffers between replays
        g.replay()
        torch.cuda.synchronize()
        got = D[:, :N]
        assert torch.equal(got, eager[:, :N]), \
            (rep, np.argwhere((got != eager[:, :N]).cpu().numpy())[:5])
