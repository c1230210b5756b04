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
//  * 256x256 output tile, 4 waves (2x2) of 128x128 outputs each;
//  * K slices of 32 (64-byte LDS rows), 5 LDS stages (160 KiB): stage kt+4 is
//    requested while stage kt is multiplied, so each load has three stages of
//    MFMA work to land;
//  * one barrier per stage; it certifies stage kt+1 (every wave waited for its
//    own loads of that stage first) and that stage kt-1 is no longer read,
//    which lets the first fragments of stage kt+1 be read during stage kt;
//  * LDS rows of 32 K-values (64 bytes) are paired into 128-byte lines whose
//    16-byte slots are XOR-permuted by a function of the line index (see
//    dma_lds_off). A load instruction fills 1 KiB of LDS in lane order, so
//    each lane fetches the global chunk that the layout places at its slot.
#pragma once

#include "gemm_mfma_impl.h"

namespace dgt {

template <int WM_, int WN_, int ATOM_>
struct DmaCfgT {
  static constexpr int BM = 256, BN = 256, BK = 32, STAGES = 5;
  static constexpr int WM = WM_, WN = WN_, THREADS = WM * WN * 64;
  using At = Atom<ATOM_>;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / At::M, TN = WTN / At::N;
  static constexpr int KSTEPS = BK / At::K;  // MFMA K sub-steps per stage
  static constexpr int CPS = At::K / 8;      // 16-byte chunks per sub-step
  static constexpr int ROW_BYTES = BK * 2;   // 64
  static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // 1 KiB load instructions per wave per operand per stage.
  static constexpr int LOADS_A = A_BYTES / 1024 / (THREADS / 64);
  static constexpr int LOADS_B = B_BYTES / 1024 / (THREADS / 64);
  static constexpr int LOADS_PER_STAGE = LOADS_A + LOADS_B;
  static constexpr int LOADS_PER_KSTEP = (LOADS_PER_STAGE + KSTEPS - 1) / KSTEPS;
  static constexpr int FRAGS = TM + TN;  // fragment reads per K sub-step
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
  // Each K sub-step has TM*TN MFMA slots; its memory operations (the
  // fragment reads and its share of the stage's loads) sit one per slot.
  static_assert(FRAGS + LOADS_PER_KSTEP <= TM * TN, "not enough MFMA slots");
};
using DmaCfg = DmaCfgT<2, 2, 32>;

// LDS layout of one operand box: rows 2L and 2L+1 (64 bytes each) share the
// 128-byte line L, whose eight 16-byte slots hold (row & 1, chunk) as
// v = ((row & 1) << 2) | chunk, placed at slot v ^ S(L). S is linear over
// GF(2) in the bits of L: bit i of S is the parity of L & kSwzMask[i].
// S(L) = (L>>1 & 1) | (L>>3 & 1) << 1 keeps each row's four chunks in its own
// 64 bytes and measured zero LDS bank conflicts on the fragment reads; the
// (r>>1)^(r>>3) chunk swizzle and three other candidates measured 2-way.
constexpr int kSwzMask0 = 0x2, kSwzMask1 = 0x8, kSwzMask2 = 0x0;
__device__ static inline int dma_line_swz(int line) {
  return (__builtin_popcount(line & kSwzMask0) & 1) |
         ((__builtin_popcount(line & kSwzMask1) & 1) << 1) |
         ((__builtin_popcount(line & kSwzMask2) & 1) << 2);
}

// Byte offset of 16-byte chunk `chunk` (0..3) of row `row` in a box.
__device__ static inline int dma_lds_off(int row, int chunk) {
  const int line = row >> 1;
  return line * 128 + (((((row & 1) << 2) | chunk) ^ dma_line_swz(line)) << 4);
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

// Per-wave addressing of the pipeline: the source offsets of this wave's load
// instructions and the LDS offsets of its fragments.
template <class C>
struct DmaPipe {
  using At = typename C::At;
  char* smem;
  // Operand bases of this tile's boxes. Kept as plain pointers (the buffer
  // resource is built at each load, which the compiler hoists): a member of
  // the device-only resource type makes this struct unusable in the host
  // compilation pass that instantiates the kernel.
  const uint16_t* baseA;
  const uint16_t* baseB;
  int wave;
  int voffA[C::LOADS_A], voffB[C::LOADS_B];
  int offA[C::KSTEPS][C::TM], offB[C::KSTEPS][C::TN];

  // Instruction i of wave w fills LDS lines 8*(w*L + i) .. +7 in lane order:
  // lane l writes slot l % 8 of line +l/8, so it fetches the (row, chunk) the
  // layout puts there. The K position advances through the scalar offset.
  __device__ inline void init(const GemmArgs& p, char* smem_, int m0, int n0, int wave_,
                              int lane, int wm, int wn) {
    smem = smem_;
    wave = wave_;
    baseA = static_cast<const uint16_t*>(p.A) + (int64_t)m0 * p.lda;
    baseB = static_cast<const uint16_t*>(p.B) + (int64_t)n0 * p.ldb;
#pragma unroll
    for (int i = 0; i < C::LOADS_A; ++i) {
      const int line = (wave * C::LOADS_A + i) * 8 + (lane >> 3);
      const int v = (lane & 7) ^ dma_line_swz(line);
      voffA[i] = (int)(((int64_t)(2 * line + (v >> 2)) * p.lda + (v & 3) * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < C::LOADS_B; ++i) {
      const int line = (wave * C::LOADS_B + i) * 8 + (lane >> 3);
      const int v = (lane & 7) ^ dma_line_swz(line);
      voffB[i] = (int)(((int64_t)(2 * line + (v >> 2)) * p.ldb + (v & 3) * 8) * 2);
    }
    const int a_row0 = wm * C::WTM + At::frag_row(lane);
    const int b_row0 = wn * C::WTN + At::frag_row(lane);
    const int koct = At::frag_koct(lane);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        offA[ks][i] = dma_lds_off(a_row0 + i * At::M, ks * C::CPS + koct);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        offB[ks][j] = C::A_BYTES + dma_lds_off(b_row0 + j * At::N, ks * C::CPS + koct);
    }
  }

  // Load instruction q (0..LOADS_PER_STAGE-1) of K stage `stage` into buffer `buf`.
  __device__ __forceinline__ void issue_one(int q, int stage, int buf) const {
    if (q < 0 || q >= C::LOADS_PER_STAGE) return;
    char* dst = smem + buf * C::STAGE_BYTES;
    const int koff = stage * C::BK * 2;
    if (q < C::LOADS_A)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(baseA),
                                               (lds_ptr_t)(dst + (wave * C::LOADS_A + q) * 1024),
                                               16, voffA[q], koff, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          make_rsrc(baseB),
          (lds_ptr_t)(dst + C::A_BYTES + (wave * C::LOADS_B + q - C::LOADS_A) * 1024), 16,
          voffB[q - C::LOADS_A], koff, 0, 0);
  }
  __device__ __forceinline__ void issue_stage(int stage, int buf) const {
#pragma unroll
    for (int q = 0; q < C::LOADS_PER_STAGE; ++q) issue_one(q, stage, buf);
  }

  // Fragment t (0..FRAGS-1) of sub-step ks, in the order the MFMA nest first
  // needs them: a[0], b[0..TN-1], a[1..TM-1].
  __device__ __forceinline__ void read_one(Frags<C>& f, int buf, int ks, int t) const {
    const char* base = smem + buf * C::STAGE_BYTES;
    if (t == 0) f.a[0] = *reinterpret_cast<const u32x4*>(base + offA[ks][0]);
    else if (t <= C::TN) f.b[t - 1] = *reinterpret_cast<const u32x4*>(base + offB[ks][t - 1]);
    else if (t < C::FRAGS)
      f.a[t - C::TN] = *reinterpret_cast<const u32x4*>(base + offA[ks][t - C::TN]);
  }
  __device__ __forceinline__ void read(Frags<C>& f, int buf, int ks) const {
#pragma unroll
    for (int t = 0; t < C::FRAGS; ++t) read_one(f, buf, ks, t);
  }
};

// One K stage of the steady state, starting with the fragments of its first
// sub-step in f[P] (P is 0 or 1). Sub-step ks multiplies f[(P+ks)&1] and fills
// f[(P+ks+1)&1] with the next sub-step's fragments (for the last sub-step: the
// first fragments of the next stage, in buffer nbuf); its MFMA slots carry,
// one behind each MFMA, those fragment reads and a share of the loads of
// stage lstage into buffer lbuf. The order is pinned instruction by
// instruction so that the MFMA pipe always has the next MFMA queued.
// EPI is unused here: it only gives every kernel instantiation its own copy,
// because this compiler's host pass rejects a second kernel (same Tag, other
// epilogue) calling a device function template specialization already
// instantiated for the first one.
template <class C, class Tag, int P, int EPI>
__device__ __forceinline__ void dma_stage(typename C::At::acc_t (&acc)[C::TM][C::TN],
                                          Frags<C>* f, const DmaPipe<C>& pipe, int buf,
                                          int nbuf, int lstage, int lbuf) {
  using At = typename C::At;
  constexpr int NR = C::FRAGS, NL = C::LOADS_PER_KSTEP;
  constexpr int PAIRS = NR < NL ? NR : NL;
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) {
    Frags<C>& src = f[(P + ks) & 1];
    Frags<C>& dst = f[(P + ks + 1) & 1];
    const bool last = ks == C::KSTEPS - 1;
#pragma unroll
    for (int q = 0; q < C::TM * C::TN; ++q) {
      acc[q / C::TN][q % C::TN] =
          At::mma(Tag{}, src.a[q / C::TN], src.b[q % C::TN], acc[q / C::TN][q % C::TN]);
      // reads and loads alternate while both remain, then the rest
      int r = -1, l = -1;
      if (q < 2 * PAIRS) {
        if ((q & 1) == 0) r = q >> 1;
        else l = q >> 1;
      } else if (NR > NL) {
        r = q - PAIRS;
      } else {
        l = q - PAIRS;
      }
      if (r >= 0 && r < NR) pipe.read_one(dst, last ? nbuf : buf, last ? 0 : ks + 1, r);
      if (l >= 0 && l < NL) pipe.issue_one(ks * NL + l, lstage, lbuf);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The configuration is a fixed alias rather than a template parameter: a
// kernel template whose configuration type is dependent got no host launch
// stub from this compiler when its body held the helper lambdas used earlier.
template <class Tag, int EPI>
__global__ void __launch_bounds__(DmaCfg::THREADS)
gemm_mfma_dma_kernel(const GemmArgs p) {
  using C = DmaCfg;
  using At = typename C::At;
  using acc_t = typename At::acc_t;
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

  DmaPipe<C> pipe;
  pipe.init(p, smem, m0, n0, wave, lane, wm, wn);

  acc_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) acc[i][j][v] = 0.0f;

  const int KT = p.K / C::BK;  // whole K slices (unmasked kernel)
  constexpr int LPS = C::LOADS_PER_STAGE;

  // Prologue: request stages 0..3, wait for stage 0 (own loads, then all).
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < KT) pipe.issue_stage(s, s);
  if (KT >= 4) wait_vmcnt<3 * LPS>();
  else if (KT == 3) wait_vmcnt<2 * LPS>();
  else if (KT == 2) wait_vmcnt<LPS>();
  else wait_vmcnt<0>();
  lds_barrier();

  Frags<C> f[2];
  pipe.read(f[0], 0, 0);

  int kt = 0, buf = 0;
  // Steady state, two stages per turn so that the fragment sets keep their
  // registers for any number of sub-steps: stage kt+5 exists, so stages kt+2
  // and kt+3 are in flight behind stage kt+1 at each barrier. Stage s lives
  // in buffer s % STAGES; stage kt+4 reuses the buffer of stage kt-1.
  constexpr int P1 = C::KSTEPS & 1;
  for (; kt + 5 < KT; kt += 2) {
    wait_vmcnt<2 * LPS>();
    lds_barrier();
    int nb = buf == C::STAGES - 1 ? 0 : buf + 1;
    int lb = buf == 0 ? C::STAGES - 1 : buf - 1;
    dma_stage<C, Tag, 0, EPI>(acc, f, pipe, buf, nb, kt + 4, lb);
    buf = nb;
    wait_vmcnt<2 * LPS>();
    lds_barrier();
    nb = buf == C::STAGES - 1 ? 0 : buf + 1;
    lb = buf == 0 ? C::STAGES - 1 : buf - 1;
    dma_stage<C, Tag, P1, EPI>(acc, f, pipe, buf, nb, kt + 5, lb);
    buf = nb;
  }
  // Last stages (at most five): at most one more stage to request.
  for (; kt < KT; ++kt) {
    const int ahead = KT - kt - 2;  // requested stages behind kt+1
    if (ahead >= 2) wait_vmcnt<2 * LPS>();
    else if (ahead == 1) wait_vmcnt<LPS>();
    else wait_vmcnt<0>();
    lds_barrier();
    const int nb = buf == C::STAGES - 1 ? 0 : buf + 1;
    if (kt + 4 < KT) pipe.issue_stage(kt + 4, buf == 0 ? C::STAGES - 1 : buf - 1);
    // f[0] holds this stage's first fragments here: each pair of steady
    // stages restores the parity and the loop below keeps it.
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      if (ks + 1 < C::KSTEPS) pipe.read(f[(ks + 1) & 1], buf, ks + 1);
      mma_step<C, Tag>(acc, f[ks & 1]);
    }
    if (kt + 1 < KT) pipe.read(f[0], nb, 0);
    buf = nb;
  }

  store_tile<C, EPI, false>(acc, p, m0 + wm * C::WTM, n0 + wn * C::WTN, lane);
}

}  // namespace dgt
