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

// Two wave groups taking turns on 128x128 tiles, both operands loaded
// straight into LDS: the phase design of the 256x256 two-group kernel
// (gemm_mfma_pingpong.h) at the ring's slot geometry. Eight waves; group g
// owns rows [64g, 64g+64) of the tile, wave w of the group the 32 columns
// [32w, 32w+32): 2x1 atoms of 32x32x16, 32 accumulator registers. With one
// wave of each group per SIMD, one wave multiplies a slice while the other
// reads the next slice's fragments and issues loads, so the matrix cores do
// not stop for the loads' waits and barriers as they do with one wave per
// SIMD.
//
// A of slice t lives in half-slot 2t % SLOTS, B in (2t+1) % SLOTS. Group 1
// loads A of slice s+AA in its memory phase for slice s, group 0 B of slice
// s+BA in its own: five half-slots (80 KiB, two workgroups per CU) with
// AA = 2, BA = 1, or, for grids of at most one tile per CU, ten (160 KiB)
// with AA = 4, BA = 3. Each refill goes into the slots of a slice whose last
// reader finished at least one phase earlier (A of s+AA replaces A of s+AA-
// SLOTS/2, read last in phase 2s; B of s+BA replaces B of s+BA-SLOTS/2, read
// last by phase 2s), and each group waits for its own loads of slice s+1
// before the barrier that ends phase 2s+2, after which slice s+1 is read.
// Edges: pieces outside the operands read as zeros (the ring operand's
// out-of-range offsets), D is stored with bounds checks.
struct Pp128Wave {  // the epilogue's view of a wave's 64x32 block
  using At = Atom<32>;
  static constexpr int TM = 2, TN = 1;
};

// s_waitcnt vmcnt(n * LOADS) and lgkmcnt(0) for a run-time n in 0..3.
template <int LOADS>
__device__ __forceinline__ void pp128_wait_slices(int n) {
  if (n >= 3) pp_wait_vm_lgkm0<3 * LOADS>();
  else if (n == 2) pp_wait_vm_lgkm0<2 * LOADS>();
  else if (n == 1) pp_wait_vm_lgkm0<LOADS>();
  else pp_wait_vm_lgkm0<0>();
}

template <class Tag, int EPI, bool AMN, bool BMN, bool DEEP>
__global__ void __launch_bounds__(2 * Ring128Cfg::THREADS, DEEP ? 1 : 2)
gemm_pp128_kernel(const GemmArgs p) {
  using C = Ring128Cfg;
  using At = typename C::At;
  using acc_t = typename At::acc_t;
  constexpr int SLOTS = DEEP ? 10 : 5, AA = DEEP ? 4 : 2, BA = DEEP ? 3 : 1;
  static_assert(AA - 1 <= 3 && BA - 1 <= 3, "pp128_wait_slices counts up to three slices");
  __shared__ __attribute__((aligned(1024))) char smem[SLOTS * C::HALF_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = wave >> 2, w = wave & 3;
  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  RingOperand<AMN, 128> a;
  RingOperand<BMN, 128> b;
  a.init(p.A, p.lda, m0, p.M, p.K, group, lane);  // atoms at rows 64 group + 32 t
  b.init(p.B, p.ldb, n0, p.N, p.K, w >> 1, lane);  // atoms at columns 64 (w/2) + 32 t
  const int boff = (w & 1) ? b.off[1] : b.off[0];  // this wave's columns 32 w .. +31

  acc_t acc[2][1];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < At::NACC; ++v) acc[i][0][v] = 0.0f;

  const int KT = (p.K + C::BK - 1) / C::BK;
  auto slot = [&](int h) { return smem + (h % SLOTS) * C::HALF_BYTES; };
  // Loads of this group issued after its loads of slice t, when the last
  // slice requested so far is `last` (in slices, at most three).
  auto after = [](int t, int last) { return last - t < 0 ? 0 : last - t; };
  // Prologue: group 1 requests A of slices 0 .. AA-1, group 0 B of slices
  // 0 .. BA-1; group 1 then waits one more barrier, which puts it a phase
  // behind.
  int alast = -1, blast = -1;
  if (group == 1) {
    for (int t = 0; t < AA && t < KT; ++t) a.issue_direct(slot(2 * t), t, w, lane);
    alast = (AA < KT ? AA : KT) - 1;
    pp128_wait_slices<C::LOADS>(after(0, alast));
  } else {
    for (int t = 0; t < BA && t < KT; ++t) b.issue_direct(slot(2 * t + 1), t, w, lane);
    blast = (BA < KT ? BA : KT) - 1;
    pp128_wait_slices<C::LOADS>(after(0, blast));
  }
  pp_barrier();
  if (group == 1) {
    pp128_wait_slices<C::LOADS>(after(1, alast));  // A of slice 1, read from phase 3 on
    pp_barrier();
  }

  u32x4 fa[C::KSTEPS][2], fb[C::KSTEPS];
  for (int s = 0; s < KT; ++s) {
    const char* sa = slot(2 * s);
    const char* sb = slot(2 * s + 1);
    // Memory phase (issue priority over the other group's MFMA stream).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      fa[ks][0] = a.read(sa, 0, ks);
      fa[ks][1] = a.read(sa, 1, ks);
      fb[ks] = RingOperand<BMN, 128>::read_at(sb, boff, ks);
    }
    if (group == 0) {
      if (s + BA < KT) {
        b.issue_direct(slot(2 * (s + BA) + 1), s + BA, w, lane);
        blast = s + BA;
      }
      pp_wait_lgkm0();
    } else {
      if (s + AA < KT) {
        a.issue_direct(slot(2 * (s + AA)), s + AA, w, lane);
        alast = s + AA;
      }
      // A of slice s+1 is needed from the next phase on.
      pp128_wait_slices<C::LOADS>(after(s + 1, alast));
    }
    pp_barrier();
    __builtin_amdgcn_s_setprio(0);
    // Compute phase.
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i][0] = At::mma(Tag{}, fa[ks][i], fb[ks], acc[i][0]);
    if (group == 0) pp128_wait_slices<C::LOADS>(after(s + 1, blast));  // B of slice s+1
    pp_barrier();
  }
  if (group == 0) pp_barrier();  // matches group 1's extra prologue barrier

  const bool inner = m0 + C::BM <= p.M && n0 + C::BN <= p.N;
  if (inner) store_tile<Pp128Wave, EPI, false>(acc, p, m0 + 64 * group, n0 + 32 * w, lane);
  else store_tile<Pp128Wave, EPI, true>(acc, p, m0 + 64 * group, n0 + 32 * w, lane);
}

template <class Tag, bool AMN, bool BMN, bool DEEP>
hipError_t launch_pp128_form(const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(2 * Ring128Cfg::THREADS);
  if (a.epi == EPI_BETA0)
    return launch_kernel(gemm_pp128_kernel<Tag, EPI_BETA0, AMN, BMN, DEEP>, grid, block, s, a);
  if (a.epi == EPI_ACC_PLUS_C)
    return launch_kernel(gemm_pp128_kernel<Tag, EPI_ACC_PLUS_C, AMN, BMN, DEEP>, grid, block, s,
                         a);
  return launch_kernel(gemm_pp128_kernel<Tag, EPI_GENERAL, AMN, BMN, DEEP>, grid, block, s, a);
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

template <class Tag, bool AMN, bool BMN, int KG, bool SRC32, bool FOLD = false, bool STG2 = false>
hipError_t launch_ring_kg_src(const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(Ring128Cfg::THREADS * KG);
  if (a.epi == EPI_BETA0)
    return launch_kernel(
        gemm_ring_kernel<128, Tag, EPI_BETA0, AMN, BMN, KG, true, SRC32, FOLD, STG2>, grid, block,
        s, a);
  if (a.epi == EPI_ACC_PLUS_C)
    return launch_kernel(
        gemm_ring_kernel<128, Tag, EPI_ACC_PLUS_C, AMN, BMN, KG, true, SRC32, FOLD, STG2>, grid,
        block, s, a);
  return launch_kernel(
      gemm_ring_kernel<128, Tag, EPI_GENERAL, AMN, BMN, KG, true, SRC32, FOLD, STG2>, grid, block,
      s, a);
}

// Float32 operands (a.src32: rounded to Tag's type as they are staged) take
// their own instantiation.
template <class Tag, bool AMN, bool BMN, int KG>
hipError_t launch_ring_kg(const GemmArgs& a, hipStream_t s) {
  if (a.src32) return launch_ring_kg_src<Tag, AMN, BMN, KG, true>(a, s);
  // Exactly one operand staged: its loads three slices ahead (two sets).
  const bool stg2 = a.stage_depth == 2 && (a.a_direct != 0) != (a.b_direct != 0);
  if constexpr (KG == 2) {
    // Rows past the last whole tile row, computed by that row's workgroups.
    if (a.mfold > 0) {
      if (stg2) return launch_ring_kg_src<Tag, AMN, BMN, KG, false, true, true>(a, s);
      return launch_ring_kg_src<Tag, AMN, BMN, KG, false, true>(a, s);
    }
  }
  if (a.mfold > 0) return hipErrorInvalidValue;  // never planned
  if (stg2) return launch_ring_kg_src<Tag, AMN, BMN, KG, false, false, true>(a, s);
  return launch_ring_kg_src<Tag, AMN, BMN, KG, false>(a, s);
}

template <class Tag, bool AMN, bool BMN>
hipError_t launch_ring(const GemmArgs& a, hipStream_t s) {
  if (a.mfold > 0 && a.ring_mode != RING_KSPLIT2) return hipErrorInvalidValue;  // never planned
  if (a.ring_mode == RING_DEEP || a.ring_mode == RING_PP || a.ring_mode == RING_PP_DEEP) {
    if (a.src32 || !a.a_direct || !a.b_direct) return hipErrorInvalidValue;  // never planned
    if (a.ring_mode == RING_PP) return launch_pp128_form<Tag, AMN, BMN, false>(a, s);
    if (a.ring_mode == RING_PP_DEEP) return launch_pp128_form<Tag, AMN, BMN, true>(a, s);
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
