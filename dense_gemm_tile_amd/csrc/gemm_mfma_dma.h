// Matrix-core GEMM with direct global->LDS staging, for the case where both
// operands are K-contiguous (A stored [M][K], B stored [N][K]) and the output
// tiles are whole (no masking).
//
// Same contraction and atom nest as the general kernel (TVM TIRx `gemm`:
// "Algorithm" steps 1-3), with the Phobos `@pipeline` idea of asynchronous
// operand staging taken to CDNA4's form: `buffer_load_dwordx4 ... lds` writes
// each lane's 16 bytes straight into LDS (no VGPR round trip, no LDS write
// instructions), so the staging depth is bounded by LDS, not registers:
//
//  * 256x256 output tile, 4 waves (2x2) of 128x128, v_mfma_f32_32x32x16;
//  * K slices of 32 (64-byte LDS rows), 5 LDS stages (160 KiB): stage kt+4 is
//    requested while stage kt is multiplied, so each load has three stages of
//    MFMA work to land;
//  * one barrier per stage; it certifies stage kt+1 (every wave waited for its
//    own loads of that stage first) and that stage kt-1 is no longer read,
//    which lets the first fragments of stage kt+1 be read during stage kt;
//  * LDS row r holds 32 K-values as four 16-byte chunks; chunk c sits at
//    position c ^ (((r >> 1) ^ (r >> 3)) & 3). A load instruction fills 1 KiB
//    of LDS in lane order, so each lane fetches the global chunk that the
//    swizzle places at its slot.
#pragma once

#include "gemm_mfma_impl.h"

namespace dgt {

struct DmaCfg {
  static constexpr int BM = 256, BN = 256, BK = 32, STAGES = 5;
  static constexpr int WM = 2, WN = 2, THREADS = 256;
  using At = Atom<32>;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / At::M, TN = WTN / At::N;
  static constexpr int KSTEPS = BK / At::K;  // 2 MFMA K sub-steps per stage
  static constexpr int ROW_BYTES = BK * 2;   // 64
  static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // 1 KiB load instructions per wave per operand per stage.
  static constexpr int LOADS_A = A_BYTES / 1024 / (THREADS / 64);
  static constexpr int LOADS_B = B_BYTES / 1024 / (THREADS / 64);
  static constexpr int LOADS_PER_STAGE = LOADS_A + LOADS_B;
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
  static_assert(KSTEPS == 2, "the stage body below is written for two K sub-steps");
};

__device__ static inline int dma_swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// Byte offset of 16-byte chunk `chunk` (0..3) of 64-byte LDS row `row`.
__device__ static inline int dma_lds_off(int row, int chunk) {
  return row * DmaCfg::ROW_BYTES + ((chunk ^ dma_swz(row)) << 4);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS accesses at the compiler level but adds no
// memory-model waits: the loads in flight to LDS are accounted for by the
// explicit vmcnt wait before it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

using lds_ptr_t = __attribute__((address_space(3))) void*;

template <class Tag, int EPI>
__global__ void __launch_bounds__(DmaCfg::THREADS)
gemm_mfma_dma_kernel(const GemmArgs p) {
  using C = DmaCfg;
  using At = C::At;
  using acc_t = At::acc_t;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN;
  const int wn = wave % C::WN;

  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;

  const uint16_t* Ap = static_cast<const uint16_t*>(p.A) + (int64_t)m0 * p.lda;
  const uint16_t* Bp = static_cast<const uint16_t*>(p.B) + (int64_t)n0 * p.ldb;
  const auto rsA = make_rsrc(Ap);
  const auto rsB = make_rsrc(Bp);

  // Per-lane source offsets of this wave's load instructions (loop-invariant;
  // the K position advances through the scalar offset). Instruction i of wave
  // w fills LDS rows 16*(w*L + i) .. +15; lane l lands in row +l/4, slot l%4.
  int voffA[C::LOADS_A], voffB[C::LOADS_B];
#pragma unroll
  for (int i = 0; i < C::LOADS_A; ++i) {
    const int row = (wave * C::LOADS_A + i) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ dma_swz(row);
    voffA[i] = (int)(((int64_t)row * p.lda + chunk * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::LOADS_B; ++i) {
    const int row = (wave * C::LOADS_B + i) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ dma_swz(row);
    voffB[i] = (int)(((int64_t)row * p.ldb + chunk * 8) * 2);
  }

  // Load instruction q (0..LOADS_PER_STAGE-1) of stage `stage` into buffer `buf`.
  auto issue_one = [&](int q, int stage, int buf) {
    if (q < 0 || q >= C::LOADS_PER_STAGE) return;
    char* dst = smem + buf * C::STAGE_BYTES;
    const int koff = stage * C::BK * 2;
    if (q < C::LOADS_A)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsA, (lds_ptr_t)(dst + (wave * C::LOADS_A + q) * 1024), 16, voffA[q], koff, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsB, (lds_ptr_t)(dst + C::A_BYTES + (wave * C::LOADS_B + q - C::LOADS_A) * 1024), 16,
          voffB[q - C::LOADS_A], koff, 0, 0);
  };
  auto issue_stage = [&](int stage, int buf) {
#pragma unroll
    for (int q = 0; q < C::LOADS_PER_STAGE; ++q) issue_one(q, stage, buf);
  };

  // Fragment addresses within a stage (bytes), one per atom and K sub-step.
  const int a_row0 = wm * C::WTM + At::frag_row(lane);
  const int b_row0 = wn * C::WTN + At::frag_row(lane);
  const int koct = At::frag_koct(lane);
  int offA[C::KSTEPS][C::TM], offB[C::KSTEPS][C::TN];
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i) offA[ks][i] = dma_lds_off(a_row0 + i * At::M, ks * 2 + koct);
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      offB[ks][j] = C::A_BYTES + dma_lds_off(b_row0 + j * At::N, ks * 2 + koct);
  }
  auto read = [&](Frags<C>& f, int buf, int ks) {
    const char* base = smem + buf * C::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) f.a[i] = *reinterpret_cast<const u32x4*>(base + offA[ks][i]);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) f.b[j] = *reinterpret_cast<const u32x4*>(base + offB[ks][j]);
  };
  // Fragment t (0..TM+TN-1) in the order the MFMA nest first needs them:
  // a[0], b[0..TN-1], a[1..TM-1].
  auto read_one = [&](Frags<C>& f, int buf, int ks, int t) {
    const char* base = smem + buf * C::STAGE_BYTES;
    if (t == 0) f.a[0] = *reinterpret_cast<const u32x4*>(base + offA[ks][0]);
    else if (t <= C::TN) f.b[t - 1] = *reinterpret_cast<const u32x4*>(base + offB[ks][t - 1]);
    else f.a[t - C::TN] = *reinterpret_cast<const u32x4*>(base + offA[ks][t - C::TN]);
  };

  acc_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) acc[i][j][v] = 0.0f;

  const int KT = p.K / C::BK;  // whole K slices (unmasked kernel)

  // Prologue: request stages 0..3, wait for stage 0 (own loads, then all).
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < KT) issue_stage(s, s);
  if (KT >= 4) wait_vmcnt<3 * C::LOADS_PER_STAGE>();
  else if (KT == 3) wait_vmcnt<2 * C::LOADS_PER_STAGE>();
  else if (KT == 2) wait_vmcnt<C::LOADS_PER_STAGE>();
  else wait_vmcnt<0>();
  lds_barrier();

  Frags<C> cur, nxt;
  read(cur, 0, 0);

  int kt = 0, buf = 0;
  // Steady state: stage kt+4 exists, so stages kt+2 and kt+3 are in flight
  // behind stage kt+1 when the barrier waits for it.
  for (; kt + 4 < KT; ++kt) {
    wait_vmcnt<2 * C::LOADS_PER_STAGE>();
    lds_barrier();
    const int nbuf = buf == C::STAGES - 1 ? 0 : buf + 1;
    const int lbuf = buf == 0 ? C::STAGES - 1 : buf - 1;  // == (kt + 4) % STAGES
    // Issue order, pinned instruction by instruction so the MFMA pipe always
    // has the next MFMA queued: in sub-step 0 (fragments `cur`) the even
    // MFMA slots read the fragments of sub-step 1 and the odd ones issue half
    // of the stage's loads; in sub-step 1 (`nxt`) the even slots read the
    // first fragments of the next stage and the odd ones issue the other half.
#pragma unroll
    for (int q = 0; q < C::TM * C::TN; ++q) {
      acc[q / C::TN][q % C::TN] =
          At::mma(Tag{}, cur.a[q / C::TN], cur.b[q % C::TN], acc[q / C::TN][q % C::TN]);
      if ((q & 1) == 0) read_one(nxt, buf, 1, q >> 1);
      else if ((q >> 1) < C::LOADS_PER_STAGE / 2) issue_one(q >> 1, kt + 4, lbuf);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < C::TM * C::TN; ++q) {
      acc[q / C::TN][q % C::TN] =
          At::mma(Tag{}, nxt.a[q / C::TN], nxt.b[q % C::TN], acc[q / C::TN][q % C::TN]);
      if ((q & 1) == 0) read_one(cur, nbuf, 0, q >> 1);
      else if ((q >> 1) < C::LOADS_PER_STAGE / 2)
        issue_one(C::LOADS_PER_STAGE / 2 + (q >> 1), kt + 4, lbuf);
      __builtin_amdgcn_sched_barrier(0);
    }
    buf = nbuf;
  }
  // Last (up to four) stages: nothing more to request.
  for (; kt < KT; ++kt) {
    const int ahead = KT - kt - 2;  // stages behind kt+1 still in flight
    if (ahead >= 2) wait_vmcnt<2 * C::LOADS_PER_STAGE>();
    else if (ahead == 1) wait_vmcnt<C::LOADS_PER_STAGE>();
    else wait_vmcnt<0>();
    lds_barrier();
    const int nbuf = buf == C::STAGES - 1 ? 0 : buf + 1;
    read(nxt, buf, 1);
    mma_step<C, Tag>(acc, cur);
    if (kt + 1 < KT) read(cur, nbuf, 0);
    mma_step<C, Tag>(acc, nxt);
    buf = nbuf;
  }

  store_tile<C, EPI, false>(acc, p, m0 + wm * C::WTM, n0 + wn * C::WTN, lane);
}

}  // namespace dgt
