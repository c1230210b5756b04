// Matrix-core GEMM for whole 256x256 output tiles whose operands are both
// K-contiguous (A stored [M][K], B stored [N][K]): direct global->LDS staging
// and two wave groups that take turns on the matrix cores.
//
// Same contraction and atom nest as the general kernel (TVM TIRx `gemm`:
// "Algorithm" steps 1-3), with the Phobos `@pipeline` idea of asynchronous
// operand staging carried to CDNA4 as follows.
//
//  * Eight waves, two groups of four. Wave w runs on SIMD w % 4, so every SIMD
//    holds one wave of each group. Group g owns output rows [128g, 128g+128)
//    of the tile, wave w within it the 64 columns [64(w%4), +64): a 128x64
//    block of 4x2 v_mfma_f32_32x32x16 atoms (128 accumulator registers, so two
//    waves fit one SIMD's register file).
//  * Time is cut into phases at workgroup barriers. In each phase one group
//    multiplies a whole K slice of 64 from registers (32 MFMAs per wave, no
//    memory instruction in between) while the other group reads its next
//    slice's 24 fragments from LDS and issues loads; the roles swap at every
//    barrier. The matrix cores of a SIMD are therefore fed by one wave while
//    the other one waits on memory.
//  * Loads are buffer_load_dwordx4 with the LDS bit: each lane's 16 bytes go
//    straight into LDS (no VGPR round trip, no LDS store instruction). One
//    instruction fills 1 KiB of LDS in lane order: eight whole 128-byte row
//    segments (64 K-values of eight rows), so every global access is a full
//    cache line.
//  * LDS is a ring of five 32 KiB half-slots; A of K slice t lives in slot
//    2t % 5 and B in slot (2t+1) % 5. One half slice (32 instructions per
//    workgroup) is loaded per phase, so the texture path is busy at an even
//    rate: group 1 loads A of slice s+2 in its memory phase for slice s,
//    group 0 loads B of slice s+1 in its own. A slot is refilled only after
//    the phase in which the second group read it, and every load has at least
//    one further phase to land before the barrier that certifies it.
//  * Rows are 128 bytes (64 K-values, eight 16-byte chunks); chunk c of row r
//    sits at chunk position c ^ ((r ^ (r>>3)) & 7), the layout that the
//    general kernel uses, which keeps the fragment reads free of bank
//    conflicts. Lane l of a load instruction covering rows r0..r0+7 writes
//    slot l%8 of row r0 + l/8, so it fetches the chunk that the layout puts
//    there.
//  * This compiler inserts no waits between a direct-to-LDS load and LDS
//    reads of the same bytes: each wave waits on vmcnt for its own loads of a
//    slice before the barrier that precedes the slice's first read.
#pragma once

#include "gemm_mfma_impl.h"

namespace dgt {

struct PingPongCfg {
  static constexpr int BM = 256, BN = 256, BK = 64;
  static constexpr int WM = 2, WN = 4, THREADS = WM * WN * 64;
  using At = Atom<32>;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // 128 x 64 per wave
  static constexpr int TM = WTM / At::M, TN = WTN / At::N;
  static constexpr int KSTEPS = BK / At::K;            // MFMA K sub-steps per slice
  static constexpr int FRAGS = KSTEPS * (TM + TN);     // fragment reads per slice
  static constexpr int ROW_BYTES = BK * 2;             // 128
  static constexpr int SLOT_BYTES = 256 * ROW_BYTES;   // one operand of one slice
  static constexpr int SLOTS = 5;
  static constexpr int LDS_BYTES = SLOTS * SLOT_BYTES;
  static constexpr int LOADS = SLOT_BYTES / 1024 / (THREADS / 64 / 2);  // per wave per half slice
  static_assert(BM == 256 && BN == 256, "slots hold 256 rows");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
  static_assert(LOADS == 8, "four waves load one 32 KiB half slice");
};

// Byte offset of 16-byte chunk `chunk` of row `row` in a slot.
__device__ static inline int pp_lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// s_waitcnt with the other counters left alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void pp_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int N>
__device__ __forceinline__ void pp_wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void pp_wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Phase boundary: a workgroup barrier that no instruction crosses in either
// direction at compile time (MFMAs included), with no memory-model waits of
// its own; the loads it certifies were waited for explicitly.
__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

using pp_lds_ptr_t = __attribute__((address_space(3))) void*;

// Per-wave addressing: the source of this wave's load instructions (A for
// group 1, B for group 0) and the LDS offsets of its fragments.
struct PingPongPipe {
  using C = PingPongCfg;
  using At = C::At;
  char* smem;
  // Base of this wave's operand box. A plain pointer (the buffer resource is
  // built at each load and hoisted by the compiler): a member of the
  // device-only resource type makes the struct unusable in the host pass.
  const uint16_t* base;
  int ld2;   // row pitch in bytes
  int row;   // byte offset of this lane's first row
  int c0;    // chunk of this lane in instruction 0
  int lw;    // wave index within its group
  int offA[C::TM], offB[C::TN];  // fragment offsets within a slot, sub-step 0

  __device__ inline void init(const GemmArgs& p, char* smem_, int m0, int n0, int group, int wave,
                              int lane, int wm, int wn) {
    smem = smem_;
    lw = wave & 3;
    if (group == 1) {
      base = static_cast<const uint16_t*>(p.A) + (int64_t)m0 * p.lda;
      ld2 = (int)(p.lda * 2);
    } else {
      base = static_cast<const uint16_t*>(p.B) + (int64_t)n0 * p.ldb;
      ld2 = (int)(p.ldb * 2);
    }
    // Instruction i of wave lw covers rows 64*lw + 8i .. +7. Lane l fills
    // slot l%8 of row 64*lw + 8i + l/8, whose swizzle is (l/8) ^ i, so it
    // fetches chunk (l%8) ^ (l/8) ^ i.
    row = (lw * 64 + (lane >> 3)) * ld2;
    c0 = (lane & 7) ^ (lane >> 3);
    // Fragment rows keep their low three bits per lane and the chunk of
    // sub-step ks is 2*ks + koct, so the offset for sub-step ks is the
    // sub-step-0 offset with ks << 5 XOR-ed in (bits 5-6 of the chunk slot).
    const int koct = At::frag_koct(lane);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      offA[i] = pp_lds_off(wm * C::WTM + i * At::M + At::frag_row(lane), koct);
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      offB[j] = pp_lds_off(wn * C::WTN + j * At::N + At::frag_row(lane), koct);
  }

  // Load instruction i (0..7) of K slice `slice` into half-slot `slot`.
  __device__ __forceinline__ void issue(int i, int slice, int slot) const {
    const int voff = row + ((c0 ^ i) << 4);
    const int soff = slice * C::ROW_BYTES + i * 8 * ld2;
    char* dst = smem + slot * C::SLOT_BYTES + (lw * C::LOADS + i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base), (pp_lds_ptr_t)dst, 16, voff, soff, 0,
                                             0);
  }
  __device__ __forceinline__ void issue_half(int slice, int slot) const {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) issue(i, slice, slot);
  }

  // All fragments of one K slice (A in slot sa, B in slot sb).
  __device__ __forceinline__ void read(Frags<C> (&f)[C::KSTEPS], int sa, int sb) const {
    const char* a = smem + sa * C::SLOT_BYTES;
    const char* b = smem + sb * C::SLOT_BYTES;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        f[ks].a[i] = *reinterpret_cast<const u32x4*>(a + (offA[i] ^ (ks << 5)));
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        f[ks].b[j] = *reinterpret_cast<const u32x4*>(b + (offB[j] ^ (ks << 5)));
    }
  }
};

// Multiply one K slice held in registers.
template <class C, class Tag>
__device__ __forceinline__ void pp_multiply(typename C::At::acc_t (&acc)[C::TM][C::TN],
                                            const Frags<C> (&f)[C::KSTEPS]) {
  using At = typename C::At;
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc[i][j] = At::mma(Tag{}, f[ks].a[i], f[ks].b[j], acc[i][j]);
}

// The phase loop. Phase numbers: the prologue is phase 0; group 0 reads slice
// s in phase 2s+1 and multiplies it in 2s+2; group 1 reads it in 2s+2 and
// multiplies it in 2s+3 (its phase 1 is idle). Slice t must be in LDS at the
// end of phase 2t and its slots are free after phase 2t+2.
//
// EPI is unused here: it gives each kernel instantiation its own copy, since
// this compiler's host pass rejects a second kernel (same Tag, other
// epilogue) calling a device function template specialization already
// instantiated for the first one.
template <class C, class Tag, int EPI>
__device__ __forceinline__ void pp_mainloop(typename C::At::acc_t (&acc)[C::TM][C::TN],
                                            const PingPongPipe& pipe, int K, int group) {
  const int KT = K / C::BK;  // whole slices (unmasked kernel)
  // Prologue: group 1 requests A of slices 0 and 1, group 0 B of slice 0.
  if (group == 1) {
    pipe.issue_half(0, 0);
    if (KT > 1) {
      pipe.issue_half(1, 2);
      pp_wait_vm<C::LOADS>();
    } else {
      pp_wait_vm<0>();
    }
  } else {
    pipe.issue_half(0, 1);
    pp_wait_vm<0>();
  }
  pp_barrier();
  if (group == 1) {
    pp_wait_vm<0>();  // A of slice 1, read from phase 3 on
    pp_barrier();
  }

  Frags<C> f[C::KSTEPS];
  PingPongPipe pp = pipe;
  int h = 0;  // (2s) % 5: the slot of A of slice s
  for (int s = 0; s < KT; ++s) {
    // Keep the per-lane address terms opaque to loop-invariant code motion,
    // so that the 8 load offsets and 24 fragment offsets are formed at use
    // instead of occupying registers next to 128 accumulators.
    asm volatile("" : "+v"(pp.c0), "+v"(pp.row));
    asm volatile("" : "+v"(pp.offA[0]), "+v"(pp.offA[1]), "+v"(pp.offA[2]), "+v"(pp.offA[3]),
                 "+v"(pp.offB[0]), "+v"(pp.offB[1]));
    const int sa = h, sb = h == 4 ? 0 : h + 1;
    // Memory phase: fragments first (they drain through LDS while the load
    // instructions queue on the texture path), then this group's half slice.
    pp.read(f, sa, sb);
    if (group == 0) {
      if (s + 1 < KT) pp.issue_half(s + 1, h >= 2 ? h - 2 : h + 3);  // B of s+1: (2s+3) % 5
      pp_wait_lgkm0();
    } else {
      const bool ld = s + 2 < KT;
      if (ld) pp.issue_half(s + 2, h >= 1 ? h - 1 : h + 4);  // A of s+2: (2s+4) % 5
      // A of slice s+1 (requested one memory phase earlier) is needed from
      // the next phase on.
      if (ld) pp_wait_vm_lgkm0<C::LOADS>();
      else pp_wait_vm_lgkm0<0>();
    }
    pp_barrier();
    // Compute phase.
    pp_multiply<C, Tag>(acc, f);
    if (group == 0) pp_wait_vm<0>();  // B of slice s+1, read from the next phase on
    pp_barrier();
    h = h >= 3 ? h - 3 : h + 2;
  }
  if (group == 0) pp_barrier();  // matches group 1's idle phase: same barrier count
}

template <class Tag, int EPI>
__global__ void __launch_bounds__(PingPongCfg::THREADS) gemm_mfma_pingpong_kernel(const GemmArgs p) {
  using C = PingPongCfg;
  using At = typename C::At;
  using acc_t = typename At::acc_t;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: no divergent barriers
  const int group = wave >> 2;
  const int wm = group, wn = wave & 3;

  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;

  PingPongPipe pipe;
  pipe.init(p, smem, m0, n0, group, wave, lane, wm, wn);

  acc_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) acc[i][j][v] = 0.0f;

  pp_mainloop<C, Tag, EPI>(acc, pipe, p.K, group);
  store_tile<C, EPI, false>(acc, p, m0 + wm * C::WTM, n0 + wn * C::WTN, lane);
}

}  // namespace dgt
