// 128x128 tiles on the ring design (gemm_ring.h): the kernel for mid-size
// shapes (too few 256x256 tiles to fill the chip), ragged shapes and operands
// whose rows are not 16-byte aligned, for f16/bf16 operands in any of the
// four layouts. Three forms: two workgroups per CU (five half-slots each),
// two K groups per workgroup, and the deep ring below for grids of at most
// one tile per CU.
#include "gemm_ring.h"

namespace dgt {

namespace {

// Deep ring: both operands loaded straight into LDS, one workgroup of 4
// waves per CU with all 160 KiB as ten half-slots (slot 2t % 10 for A of
// slice t, 2t+1 for B). For grids of at most one tile per CU, where no second
// workgroup shares the CU.
//
// With one wave per SIMD nothing else hides a fragment read's latency, so the
// loop is pipelined across slices: iteration s multiplies slice s from
// registers while it reads slice s+1's fragments from LDS, and every slice
// is requested five slices before it is multiplied. One barrier per slice
// certifies slice s+1 (each wave waited for its own loads of it) and frees
// slice s's slots (every wave read it in the previous iteration), which
// then take slice s+5. Measured against reading each k-step's fragments just
// before its MFMAs: 4 % faster at 2048^3 NN with C, equal on NT shapes, whose
// slices take about 0.58 us against 0.26 us of MFMA work either way (1, 2 or
// 3 slices of lookahead change nothing there either).
template <class Tag, int EPI, bool AMN, bool BMN>
__global__ void __launch_bounds__(Ring128Cfg::THREADS, 1)
gemm_ring128_deep_kernel(const GemmArgs p) {
  using C = Ring128Cfg;
  using At = typename C::At;
  using acc_t = typename At::acc_t;
  constexpr int SLOTS = 10, AHEAD = SLOTS / 2 - 1;  // slices in flight behind the next
  __shared__ __attribute__((aligned(1024))) char smem[SLOTS * C::HALF_BYTES];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  RingOperand<AMN, 128> a;
  RingOperand<BMN, 128> b;
  a.init(p.A, p.lda, m0, p.M, p.K, wm, lane);
  b.init(p.B, p.ldb, n0, p.N, p.K, wn, lane);

  acc_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) acc[i][j][v] = 0.0f;

  const int KT = (p.K + C::BK - 1) / C::BK;
  auto slot = [&](int h) { return smem + (h % SLOTS) * C::HALF_BYTES; };
  auto request = [&](int t) {
    a.issue_direct(slot(2 * t), t, w, lane);
    b.issue_direct(slot(2 * t + 1), t, w, lane);
  };

  // Interior tiles that read C request it right after the prologue's loads
  // (64 registers per lane), so it arrives while the K loop runs.
  constexpr bool PRE_C = EPI != EPI_BETA0;
  const bool inner = m0 + C::BM <= p.M && n0 + C::BN <= p.N;
  const bool pre_c = PRE_C && p.wide_epi && inner;
  WideC<C> cpre;
  constexpr int NC = PRE_C ? C::TM * C::TN * At::NACC / 4 : 0;  // C loads per lane

  // Wait until this wave's loads of slice t have landed (and its LDS reads
  // are done). Loads are issued in the order slices 0..AHEAD, C (pre_c),
  // then slice AHEAD+1+j in iteration j; the ones issued after slice t may
  // stay in flight: `after` slices, and the C loads when t <= AHEAD.
  auto wait_for = [&](int t, int issued_last) {
    int after = issued_last - t;
    after = after < 0 ? 0 : (after > AHEAD ? AHEAD : after);
    const bool c_after = pre_c && t <= AHEAD;
    constexpr int L2 = 2 * C::LOADS;
    if (c_after) {
      if (after >= 4) pp_wait_vm_lgkm0<4 * L2 + NC>();
      else if (after == 3) pp_wait_vm_lgkm0<3 * L2 + NC>();
      else if (after == 2) pp_wait_vm_lgkm0<2 * L2 + NC>();
      else if (after == 1) pp_wait_vm_lgkm0<L2 + NC>();
      else pp_wait_vm_lgkm0<NC>();
    } else {
      if (after >= 4) pp_wait_vm_lgkm0<4 * L2>();
      else if (after == 3) pp_wait_vm_lgkm0<3 * L2>();
      else if (after == 2) pp_wait_vm_lgkm0<2 * L2>();
      else if (after == 1) pp_wait_vm_lgkm0<L2>();
      else pp_wait_vm_lgkm0<0>();
    }
  };
  static_assert(AHEAD == 4, "wait_for counts at most four slices in flight behind the next");
  static_assert(4 * 2 * C::LOADS + NC < 64, "vmcnt is a 6-bit counter");

  auto read_slice = [&](u32x4 (&fa)[C::KSTEPS][C::TM], u32x4 (&fb)[C::KSTEPS][C::TN], int t) {
    const char* sa = slot(2 * t);
    const char* sb = slot(2 * t + 1);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) fa[ks][i] = a.read(sa, i, ks);
#pragma unroll
      for (int j = 0; j < C::TN; ++j) fb[ks][j] = b.read(sb, j, ks);
    }
  };
  auto multiply = [&](const u32x4 (&fa)[C::KSTEPS][C::TM], const u32x4 (&fb)[C::KSTEPS][C::TN]) {
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = At::mma(Tag{}, fa[ks][i], fb[ks][j], acc[i][j]);
  };

  // Prologue: slices 0 .. AHEAD (all ten half-slots), then C; slice 0 read.
  const int pro = KT - 1 < AHEAD ? KT - 1 : AHEAD;  // last slice requested
  for (int t = 0; t <= pro; ++t) request(t);
  if constexpr (PRE_C) {
    if (pre_c) load_wide_c<C>(cpre, p, m0 + wm * C::WTM, n0 + wn * C::WTN, lane);
  }
  wait_for(0, pro);
  pp_barrier();
  u32x4 fa0[C::KSTEPS][C::TM], fb0[C::KSTEPS][C::TN];
  u32x4 fa1[C::KSTEPS][C::TM], fb1[C::KSTEPS][C::TN];
  read_slice(fa0, fb0, 0);

  // One step: multiply slice s (in cur), read slice s+1 into nxt. `last` is
  // the last slice requested before this step.
  auto step = [&](int s, int& last, u32x4 (&ca)[C::KSTEPS][C::TM], u32x4 (&cb)[C::KSTEPS][C::TN],
                  u32x4 (&na)[C::KSTEPS][C::TM], u32x4 (&nb)[C::KSTEPS][C::TN]) {
    if (s + 1 < KT) {
      wait_for(s + 1, last);
      pp_barrier();
      if (s + AHEAD + 1 < KT) {
        request(s + AHEAD + 1);  // into slice s's slots
        last = s + AHEAD + 1;
      }
      read_slice(na, nb, s + 1);
    }
    multiply(ca, cb);
  };
  int last = pro;
  int s = 0;
  for (; s + 1 < KT; s += 2) {
    step(s, last, fa0, fb0, fa1, fb1);
    step(s + 1, last, fa1, fb1, fa0, fb0);
  }
  if (s < KT) step(s, last, fa0, fb0, fa1, fb1);

  if (inner) store_tile<C, EPI, false>(acc, p, m0 + wm * C::WTM, n0 + wn * C::WTN, lane, cpre, pre_c);
  else store_tile<C, EPI, true>(acc, p, m0 + wm * C::WTM, n0 + wn * C::WTN, lane);
}

template <class Tag, bool AMN, bool BMN>
hipError_t launch_ring_deep(const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(Ring128Cfg::THREADS);
  if (a.epi == EPI_BETA0)
    return launch_kernel(gemm_ring128_deep_kernel<Tag, EPI_BETA0, AMN, BMN>, grid, block, s, a);
  if (a.epi == EPI_ACC_PLUS_C)
    return launch_kernel(gemm_ring128_deep_kernel<Tag, EPI_ACC_PLUS_C, AMN, BMN>, grid, block, s,
                         a);
  return launch_kernel(gemm_ring128_deep_kernel<Tag, EPI_GENERAL, AMN, BMN>, grid, block, s, a);
}

template <class Tag, bool AMN, bool BMN, int KG, bool SRC32>
hipError_t launch_ring_kg_src(const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(Ring128Cfg::THREADS * KG);
  if (a.epi == EPI_BETA0)
    return launch_kernel(gemm_ring_kernel<128, Tag, EPI_BETA0, AMN, BMN, KG, true, SRC32>, grid,
                         block, s, a);
  if (a.epi == EPI_ACC_PLUS_C)
    return launch_kernel(gemm_ring_kernel<128, Tag, EPI_ACC_PLUS_C, AMN, BMN, KG, true, SRC32>,
                         grid, block, s, a);
  return launch_kernel(gemm_ring_kernel<128, Tag, EPI_GENERAL, AMN, BMN, KG, true, SRC32>, grid,
                       block, s, a);
}

// Float32 operands (a.src32: rounded to Tag's type as they are staged) take
// their own instantiation.
template <class Tag, bool AMN, bool BMN, int KG>
hipError_t launch_ring_kg(const GemmArgs& a, hipStream_t s) {
  if (a.src32) return launch_ring_kg_src<Tag, AMN, BMN, KG, true>(a, s);
  return launch_ring_kg_src<Tag, AMN, BMN, KG, false>(a, s);
}

template <class Tag, bool AMN, bool BMN>
hipError_t launch_ring(const GemmArgs& a, hipStream_t s) {
  if (a.ring_mode == RING_DEEP) {
    if (a.src32 || !a.a_direct || !a.b_direct) return hipErrorInvalidValue;  // never planned
    return launch_ring_deep<Tag, AMN, BMN>(a, s);
  }
  if (a.ring_mode == RING_KSPLIT2) return launch_ring_kg<Tag, AMN, BMN, 2>(a, s);
  return launch_ring_kg<Tag, AMN, BMN, 1>(a, s);
}

template <class Tag>
hipError_t launch_ring_layout(bool ta, bool tb, const GemmArgs& a, hipStream_t s) {
  // A is M-contiguous when stored transposed; B is N-contiguous when not.
  if (!ta && tb) return launch_ring<Tag, false, false>(a, s);
  if (!ta && !tb) return launch_ring<Tag, false, true>(a, s);
  if (ta && tb) return launch_ring<Tag, true, false>(a, s);
  return launch_ring<Tag, true, true>(a, s);
}

}  // namespace

hipError_t launch_ring128(int dtype, bool ta, bool tb, const GemmArgs& a, hipStream_t s) {
  if (dtype == 0) return launch_ring_layout<TagF16>(ta, tb, a, s);
  return launch_ring_layout<TagBF16>(ta, tb, a, s);
}

}  // namespace dgt
