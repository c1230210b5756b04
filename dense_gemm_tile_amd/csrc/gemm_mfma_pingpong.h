// Matrix-core GEMM for 256x256 output tiles: direct global->LDS staging and
// two wave groups that take turns on the matrix cores. Each operand may be
// K-contiguous (A stored [M][K], B stored [N][K]) or M/N-contiguous (A stored
// [K][M], B stored [K][N]). Whole tiles, or (MASK) edge tiles and K tails
// whose operands still load in whole 16-byte pieces.
//
// Same contraction and atom nest as the general kernel (TVM TIRx `gemm`:
// "Algorithm" steps 1-3), with the Phobos `@pipeline` idea of asynchronous
// operand staging carried to CDNA4 as follows.
//
//  * Eight waves, two groups of four. Wave w runs on SIMD w % 4, so every SIMD
//    holds one wave of each group. Group g owns output rows [128g, 128g+128)
//    of the tile, wave w within it the 64 columns [64(w%4), +64): a 128x64
//    block of atoms (128 accumulator registers, so two waves fit one SIMD's
//    register file). The atom is v_mfma_f32_16x16x32 (8x4 of them) when A is
//    K-contiguous and v_mfma_f32_32x32x16 (4x2) when A is M-contiguous. Both
//    give the same sums bit for bit here; the chip runs this kernel at its
//    power limit, and the 16x16x32 form draws less power per cycle, so it
//    clocks higher: measured +5% at 8192^3 with B [N][K], +3% with B [K][N],
//    but -1 to -5% when A is [K][M], whose transposed fragment reads then
//    wait longer.
//  * Time is cut into phases at workgroup barriers. In each phase one group
//    multiplies a whole K slice of 64 from registers (32 MFMAs per wave, no
//    memory instruction in between) while the other group reads its next
//    slice's fragments from LDS and issues loads; the roles swap at every
//    barrier. The matrix cores of a SIMD are therefore fed by one wave while
//    the other one waits on memory.
//  * Loads are buffer_load_dwordx4 with the LDS bit: each lane's 16 bytes go
//    straight into LDS (no VGPR round trip, no LDS store instruction). One
//    instruction fills 1 KiB of LDS in lane order, and always covers whole
//    128-byte lines of the operand in memory.
//  * LDS is a ring of five 32 KiB half-slots; A of K slice t lives in slot
//    2t % 5 and B in slot (2t+1) % 5. One half slice (32 instructions per
//    workgroup) is loaded per phase, so the texture path is busy at an even
//    rate: group 1 loads A of slice s+2 in its memory phase for slice s,
//    group 0 loads B of slice s+1 in its own. A slot is refilled only after
//    the phase in which the second group read it, and every load has at least
//    one further phase to land before the barrier that certifies it.
//  * K-contiguous operand slot: 256 rows (M or N) of 128 bytes (64 K-values,
//    eight 16-byte chunks); chunk c of row r sits at chunk position c ^ s(r).
//    A fragment (8 consecutive K-values of one row) is one ds_read_b128. For
//    the 32x32x16 atom s(r) = (r ^ (r>>3)) & 7, as in the general kernel; the
//    16x16x32 atom reads 16 rows x 4 chunks per instruction instead of 32 x
//    2, which that swizzle serves with 2-way bank conflicts (measured), so it
//    uses s(r) = r1 | (r0 ^ r3) << 1 | r2 << 2 (ri: bit i of r), chosen to be
//    conflict-free under every lane grouping of the LDS that agrees with the
//    conflict counts measured for both atoms, and measured conflict-free.
//  * M/N-contiguous operand slot: 64 rows (K) of 512 bytes (256 M or N values,
//    32 chunks); chunk c of row r sits at c ^ (4 * (r & 3)), and for the
//    16x16x32 atom also ^ (2 * r3). A fragment is two ds_read_b64_tr_b16: in
//    each group of 16 lanes, lane s names 4 consecutive values of row s/4, and
//    lane i receives value i of the group's 16 columns from each of the four
//    rows, i.e. 4 consecutive K-values of one column. The swizzle spreads the
//    rows that 32 lanes read over all banks (rows 0-3 and 0-3 of the next 16
//    columns for the 32-wide atom, rows 0-3 and 8-11 of the same 16 columns
//    for the 16-wide one).
//  * This compiler inserts no waits between a direct-to-LDS load and LDS
//    reads of the same bytes: each wave waits on vmcnt for its own loads of a
//    slice before the barrier that precedes the slice's first read.
#pragma once

#include "gemm_mfma_impl.h"

namespace dgt {

template <int ATOM>
struct PingPongCfgT {
  static constexpr int BM = 256, BN = 256, BK = 64;
  static constexpr int WM = 2, WN = 4, THREADS = WM * WN * 64;
  using At = Atom<ATOM>;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // 128 x 64 per wave
  static constexpr int TM = WTM / At::M, TN = WTN / At::N;
  static constexpr int KSTEPS = BK / At::K;            // MFMA K sub-steps per slice
  static constexpr int SLOT_BYTES = 256 * BK * 2;      // one operand of one slice
  static constexpr int SLOTS = 5;
  static constexpr int LDS_BYTES = SLOTS * SLOT_BYTES;
  static constexpr int LOADS = SLOT_BYTES / 1024 / (THREADS / 64 / 2);  // per wave per half slice
  static_assert(BM == 256 && BN == 256, "slots hold 256 rows or columns");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
  static_assert(LOADS == 8, "four waves load one 32 KiB half slice");
};
// The 1-byte-operand and float32-operand kernels use the 32x32 layout.
using PingPongCfg = PingPongCfgT<32>;

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

// Out-of-range buffer offset: loads through it read zeros.
constexpr int kOutOfRange = (int)0x80000000u;

// A buffer resource over `base` whose record count is `nrec` bytes: offsets
// at or past it read as zero.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc_n(const void* base, unsigned nrec) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nrec,
                                           0x00020000);
}

// Record count for a resource based at `b` over an operand that starts at
// `X` and whose stored extent is `ext` bytes: up to the end of the dword
// (in memory, 4-byte aligned) that holds the operand's last byte, at most
// 2^31 - 4 bytes.
__device__ inline unsigned nrec_from(const char* X, int64_t ext, const char* b) {
  const uintptr_t end = ((uintptr_t)X + (uintptr_t)ext + 3) & ~(uintptr_t)3;
  const int64_t n = (int64_t)(end - (uintptr_t)b);
  if (n <= 0) return 0u;
  return n > 0x7FFFFFFC ? 0x7FFFFFFCu : (unsigned)n;
}

typedef short pp_i16x4 __attribute__((ext_vector_type(4)));

// One operand's loads (by the wave group that loads it) and fragment reads
// (by every wave). MN: the operand is stored with M (or N) contiguous.
// NFRAG atoms of ATOM rows/columns per wave, starting at row0 of the tile.
// MASK (edge tiles): every piece is addressed through the voffset alone
// from a resource that ends at the operand's last byte, and pieces in rows
// (K-rows) past the operand or starting past its contiguous dimension get an
// out-of-range offset, so they read as zeros; the contiguous dimension must
// fill whole 16-byte pieces (the M/N-contiguous form: 16-bit elements, a
// multiple of 8).
template <bool MN, int NFRAG, int ATOM = 32, bool MASK = false>
struct PpOperand;

template <int NFRAG, int ATOM, bool MASK>
struct PpOperand<false, NFRAG, ATOM, MASK> {
  using C = PingPongCfgT<ATOM>;
  using At = typename C::At;
  // Load side: this lane's byte offset for instruction 0 and its chunk (for
  // the 16-wide atom, c1 for the odd instructions).
  const char* base;      // tile's first row (M or N index), K = 0
  int ld2, row, c0, c1;  // ld2: row pitch in bytes
  int rmask, kbytes;     // (MASK) bit i: instruction i's row is inside the operand; bytes
  unsigned nrec;         //    of K in a row; bytes from base to the operand's end
  // Read side: byte offset of each atom's fragment within a slot, sub-step 0.
  int off[NFRAG];

  __device__ static inline int swz(int r) {
    if constexpr (ATOM == 16) return ((r >> 1) & 1) | (((r ^ (r >> 3)) & 1) << 1) | (r & 4);
    else return (r ^ (r >> 3)) & 7;
  }
  __device__ static inline int lds_off(int r, int chunk) {
    return r * 128 + ((chunk ^ swz(r)) << 4);
  }
  // esz: bytes per element (2 for f16/bf16; 1 for the 1-byte-operand
  // kernels, whose 128-byte rows hold 128 K-values).
  __device__ inline void init_load(const void* X, int64_t ld, int r0, int lw, int lane,
                                   int esz = 2) {
    base = static_cast<const char*>(X) + (int64_t)r0 * ld * esz;
    ld2 = (int)(ld * esz);
    // Instruction i of wave lw covers rows 64*lw + 8i .. +7. Lane l fills
    // chunk slot l%8 of row r = 64*lw + 8i + l/8, so it fetches chunk
    // (l%8) ^ s(r) of that row: for the 32-wide atom s(r) = (l/8) ^ i, for
    // the 16-wide one s depends on r & 15 = 8(i&1) + l/8.
    row = (lw * 64 + (lane >> 3)) * ld2;
    if constexpr (ATOM == 16) {
      c0 = (lane & 7) ^ swz(lane >> 3);
      c1 = (lane & 7) ^ swz(8 + (lane >> 3));
    } else {
      c0 = (lane & 7) ^ (lane >> 3);
      c1 = 0;
    }
  }
  // (MASK) the operand's extent from this tile: rlim rows (M or N), kb
  // bytes of K values per row (a multiple of 16).
  __device__ inline void set_limits(int r0, int rlim, int kb, int lw, int lane) {
    const int rix = lw * 64 + (lane >> 3), rrem = rlim - r0;
    rmask = 0;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) rmask |= (rix + 8 * i < rrem) << i;
    kbytes = kb;
    const int64_t n = rrem > 0 ? (int64_t)(rrem - 1) * ld2 + kb : 0;
    nrec = n > 0x7FFFFFFC ? 0x7FFFFFFCu : (unsigned)n;
  }
  __device__ __forceinline__ void issue(char* slot, int lw, int i, int slice) const {
    const int chunk = ATOM == 16 ? ((i & 1) ? c1 : c0) : c0 ^ i;
    if constexpr (!MASK) {
      const int voff = row + (chunk << 4);
      const int soff = slice * 128 + i * 8 * ld2;  // a slice is 128 bytes of each row
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base), (pp_lds_ptr_t)(slot + (lw * 8 + i) * 1024),
                                               16, voff, soff, 0, 0);
    } else {
      const int kb = slice * 128 + (chunk << 4);  // the piece's first byte in its row
      const int voff = ((rmask >> i) & 1) && kb < kbytes ? row + i * 8 * ld2 + kb : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc_n(base, nrec),
                                               (pp_lds_ptr_t)(slot + (lw * 8 + i) * 1024), 16, voff,
                                               0, 0, 0);
    }
  }
  __device__ inline void init_read(int row0, int lane) {
    // The chunk of sub-step ks is (K / 8) * ks + koct, whose sub-step term
    // only touches chunk bits the lane's own koct leaves clear, so sub-step ks
    // is the sub-step-0 offset with that term XOR-ed in (byte bits 5-6 for
    // the 32-wide atom, bit 6 for the 16-wide one).
#pragma unroll
    for (int t = 0; t < NFRAG; ++t)
      off[t] = lds_off(row0 + t * At::M + At::frag_row(lane), At::frag_koct(lane));
  }
  __device__ __forceinline__ u32x4 read(const char* slot, int t, int ks) const {
    return *reinterpret_cast<const u32x4*>(slot + (off[t] ^ (ks << (ATOM == 16 ? 6 : 5))));
  }
};

template <int NFRAG, int ATOM, bool MASK>
struct PpOperand<true, NFRAG, ATOM, MASK> {
  using C = PingPongCfgT<ATOM>;
  static constexpr int NV = ATOM == 16 ? 4 : 2;  // distinct load offsets
  const uint16_t* base;  // tile's first column (M or N index), K = 0
  int64_t ld;
  int voff[NV];          // by instruction i: i & 1 (and i >= 4 for the 16-wide atom)
  int off[NFRAG];
  int cmask;             // (MASK) bit q: the piece of voff[q] starts inside the operand;
  int crem, krem0, klim; //    columns left from the tile's first; K - this lane's first
                         //    K row of slice 0; K

  // Chunk swizzle of K row r of a slot.
  __device__ static inline int swz(int r) {
    return ATOM == 16 ? (4 * (r & 3)) ^ (2 * ((r >> 3) & 1)) : 4 * (r & 3);
  }
  __device__ inline void init_load(const uint16_t* X, int64_t ld_, int c0, int lw, int lane) {
    base = X + c0;
    ld = ld_;
    // Instruction i of wave lw covers K rows 16*lw + 2i and +1 (512 bytes
    // each). Lane l fills chunk slot l%32 of row r = 16*lw + 2i + l/32, so it
    // fetches chunk (l%32) ^ swz(r) of that row; swz(r) depends on i & 1 and
    // (16-wide atom) on i >= 4, which set r & 3 and bit 3 of r.
    const int hi = lane >> 5, p = lane & 31;
#pragma unroll
    for (int q = 0; q < NV; ++q)
      voff[q] = (int)((lw * 16 + hi) * ld * 2) + ((p ^ swz(2 * (q & 1) + hi + 8 * (q >> 1))) << 4);
  }
  // (MASK) the operand's extent from this tile: clim columns (M or N), K.
  __device__ inline void set_limits(int c0, int clim, int K, int lw, int lane) {
    const int hi = lane >> 5, p = lane & 31;
    crem = clim - c0;
    cmask = 0;
#pragma unroll
    for (int q = 0; q < NV; ++q)
      cmask |= (8 * (p ^ swz(2 * (q & 1) + hi + 8 * (q >> 1))) < crem) << q;
    krem0 = K - 16 * lw - hi;
    klim = K;
  }
  // (MASK) record count from the slice's base to the end of the operand's
  // last K row's valid columns.
  __device__ inline unsigned nrec_slice(int slice) const {
    const int64_t n = 2 * ((int64_t)(klim - 1 - slice * C::BK) * ld + crem);
    return n <= 0 ? 0u : (n > 0x7FFFFFFC ? 0x7FFFFFFCu : (unsigned)n);
  }
  __device__ __forceinline__ void issue(char* slot, int lw, int i, int slice) const {
    // The slice's first K row is folded into the resource base so that the
    // 32-bit offsets stay within 16 rows of the operand.
    const uint16_t* b = base + (int64_t)slice * C::BK * ld;
    const int q = ATOM == 16 ? (i & 1) | ((i >= 4) << 1) : (i & 1);
    if constexpr (!MASK) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(b), (pp_lds_ptr_t)(slot + (lw * 8 + i) * 1024),
                                               16, voff[q], (int)(2 * i * ld * 2), 0, 0);
    } else {
      // This lane's K row is slice*64 + 16 lw + 2 i + l/32.
      const int krem = krem0 - slice * C::BK - 2 * i;
      const int voffm = (krem > 0 && ((cmask >> q) & 1)) ? voff[q] + (int)(2 * i * ld * 2)
                                                         : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc_n(b, nrec_slice(slice)),
                                               (pp_lds_ptr_t)(slot + (lw * 8 + i) * 1024), 16, voffm,
                                               0, 0, 0);
    }
  }
  __device__ inline void init_read(int col0, int lane) {
    // Lane l (group g = l/16, s = l%16) of the first transposed read of
    // sub-step 0 names row r, columns c .. c+3 of its atom, with
    //   32-wide atom: r = 8*(l/32) + s/4, c = 16*(g&1) + 4*(s%4);
    //   16-wide atom: r = 8*g + s/4,      c = 4*(s%4).
    // The second read is 4 rows down, sub-step ks is K*ks rows down: both
    // keep r & 3 and bit 3 of r, so they are immediate offsets.
    const int r = ATOM == 16 ? 8 * (lane >> 4) + ((lane & 15) >> 2)
                             : 8 * (lane >> 5) + ((lane & 15) >> 2);
#pragma unroll
    for (int t = 0; t < NFRAG; ++t) {
      const int col = ATOM == 16 ? col0 + t * 16 + 4 * (lane & 3)
                                 : col0 + t * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      off[t] = r * 512 + (((col >> 3) ^ swz(r)) << 4) + ((col & 7) << 1);
    }
  }
  __device__ __forceinline__ u32x4 read(const char* slot, int t, int ks) const {
    typedef __attribute__((address_space(3))) pp_i16x4 lds_i16x4;
    const char* p = slot + off[t] + ks * C::At::K * 512;
    const pp_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    const pp_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * 512));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  }
};

// Multiply one K slice held in registers. The K sub-steps of one accumulator
// are issued back to back (each accumulator still sums its sub-steps in K
// order, so the result is the same): a 16x16 MFMA whose accumulator input is
// the previous MFMA's output takes it without a register read, while one that
// reads another accumulator costs measurably more. Timed on gfx950 with one
// wave per SIMD: 16.2 cycles per v_mfma_f32_16x16x32_bf16 in a dependent
// chain, 18.4-19.1 cycles when 8-16 accumulators rotate; at 8192^3 the paired
// order is 3 % faster. The scheduling barrier keeps the compiler from
// interleaving the pairs again. The 32x32x16 atom showed no such cost (32.1
// vs 32.5 cycles) and keeps the sub-step-major order, which measured 1 %
// faster for it.
template <class C, class Tag>
__device__ __forceinline__ void pp_multiply(typename C::At::acc_t (&acc)[C::TM][C::TN],
                                            const Frags<C> (&f)[C::KSTEPS]) {
  using At = typename C::At;
  if constexpr (At::M == 16) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
          acc[i][j] = At::mma(Tag{}, f[ks].a[i], f[ks].b[j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
      }
  } else {
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = At::mma(Tag{}, f[ks].a[i], f[ks].b[j], acc[i][j]);
  }
}

template <bool AMN, bool BMN, int ATOM, bool MASK = false>
struct PingPongPipe {
  using C = PingPongCfgT<ATOM>;
  char* smem;
  int lw;  // wave index within its group
  PpOperand<AMN, C::TM, ATOM, MASK> a;
  PpOperand<BMN, C::TN, ATOM, MASK> b;

  __device__ inline void init(const GemmArgs& p, char* smem_, int m0, int n0, int group, int wave,
                              int lane, int wm, int wn) {
    smem = smem_;
    lw = wave & 3;
    // Only group 1 loads A and only group 0 loads B; both are set up so that
    // every register the loop keeps is defined.
    a.init_load(static_cast<const uint16_t*>(p.A), p.lda, m0, lw, lane);
    b.init_load(static_cast<const uint16_t*>(p.B), p.ldb, n0, lw, lane);
    if constexpr (MASK) {
      if constexpr (AMN) a.set_limits(m0, p.M, p.K, lw, lane);
      else a.set_limits(m0, p.M, 2 * p.K, lw, lane);
      if constexpr (BMN) b.set_limits(n0, p.N, p.K, lw, lane);
      else b.set_limits(n0, p.N, 2 * p.K, lw, lane);
    }
    a.init_read(wm * C::WTM, lane);
    b.init_read(wn * C::WTN, lane);
  }
  // This wave's eight instructions of A (group 1) or B (group 0) of a slice.
  __device__ __forceinline__ void issue_a(int slice, int slot) const {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) a.issue(smem + slot * C::SLOT_BYTES, lw, i, slice);
  }
  __device__ __forceinline__ void issue_b(int slice, int slot) const {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) b.issue(smem + slot * C::SLOT_BYTES, lw, i, slice);
  }
  // All fragments of one K slice (A in slot sa, B in slot sb).
  __device__ __forceinline__ void read(Frags<C> (&f)[C::KSTEPS], int sa, int sb) const {
    const char* pa = smem + sa * C::SLOT_BYTES;
    const char* pb = smem + sb * C::SLOT_BYTES;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) f[ks].a[i] = a.read(pa, i, ks);
#pragma unroll
      for (int j = 0; j < C::TN; ++j) f[ks].b[j] = b.read(pb, j, ks);
    }
  }
  // Keep the per-lane address terms opaque to loop-invariant code motion, so
  // that the load and fragment offsets are formed at use instead of
  // occupying registers next to 128 accumulators.
  __device__ __forceinline__ void launder() {
#pragma unroll
    for (int t = 0; t < C::TM; ++t) asm volatile("" : "+v"(a.off[t]));
#pragma unroll
    for (int t = 0; t < C::TN; ++t) asm volatile("" : "+v"(b.off[t]));
    launder_operand<AMN>(a);
    launder_operand<BMN>(b);
  }
  template <bool MN, class Op>
  __device__ __forceinline__ static void launder_operand(Op& x) {
    if constexpr (MN) {
#pragma unroll
      for (int q = 0; q < Op::NV; ++q) asm volatile("" : "+v"(x.voff[q]));
      if constexpr (MASK) asm volatile("" : "+v"(x.cmask), "+v"(x.krem0));
    } else {
      asm volatile("" : "+v"(x.row), "+v"(x.c0));
      if constexpr (ATOM == 16) asm volatile("" : "+v"(x.c1));
      if constexpr (MASK) asm volatile("" : "+v"(x.rmask));
    }
  }
};

// The phase loop. Phase numbers: the prologue is phase 0; group 0 reads slice
// s in phase 2s+1 and multiplies it in 2s+2; group 1 reads it in 2s+2 and
// multiplies it in 2s+3 (its phase 1 is idle). Slice t must be in LDS at the
// end of phase 2t and its slots are free after phase 2t+2.
//
// EPI is unused here: it gives each kernel instantiation its own copy, since
// this compiler's host pass rejects a second kernel (same Tag, other
// epilogue) calling a device function template specialization already
// instantiated for the first one.
template <class C, class Tag, int EPI, bool AMN, bool BMN, bool MASK>
__device__ __forceinline__ void pp_mainloop(typename C::At::acc_t (&acc)[C::TM][C::TN],
                                            const PingPongPipe<AMN, BMN, C::At::M, MASK>& pipe,
                                            int K, int group) {
  // Slices: whole ones, or (edge tiles) the last one cut short and zero-filled.
  const int KT = MASK ? (K + C::BK - 1) / C::BK : K / C::BK;
  // Prologue: group 1 requests A of slices 0 and 1, group 0 B of slice 0.
  if (group == 1) {
    pipe.issue_a(0, 0);
    if (KT > 1) {
      pipe.issue_a(1, 2);
      pp_wait_vm<C::LOADS>();
    } else {
      pp_wait_vm<0>();
    }
  } else {
    pipe.issue_b(0, 1);
    pp_wait_vm<0>();
  }
  pp_barrier();
  if (group == 1) {
    pp_wait_vm<0>();  // A of slice 1, read from phase 3 on
    pp_barrier();
  }

  Frags<C> f[C::KSTEPS];
  PingPongPipe<AMN, BMN, C::At::M, MASK> pp = pipe;
  int h = 0;  // (2s) % 5: the slot of A of slice s
  for (int s = 0; s < KT; ++s) {
    pp.launder();
    const int sa = h, sb = h == 4 ? 0 : h + 1;
    // Memory phase: fragments first (they drain through LDS while the load
    // instructions queue on the texture path), then this group's half slice.
    // The memory-phase wave takes issue priority over the other group's wave
    // on its SIMD (s_setprio; measured +0.8 % at 8192^3), so its reads and
    // loads are not held back behind the MFMA stream.
    __builtin_amdgcn_s_setprio(1);
    pp.read(f, sa, sb);
    if (group == 0) {
      if (s + 1 < KT) pp.issue_b(s + 1, h >= 2 ? h - 2 : h + 3);  // B of s+1: (2s+3) % 5
      pp_wait_lgkm0();
    } else {
      const bool ld = s + 2 < KT;
      if (ld) pp.issue_a(s + 2, h >= 1 ? h - 1 : h + 4);  // A of s+2: (2s+4) % 5
      // A of slice s+1 (requested one memory phase earlier) is needed from
      // the next phase on.
      if (ld) pp_wait_vm_lgkm0<C::LOADS>();
      else pp_wait_vm_lgkm0<0>();
    }
    pp_barrier();
    __builtin_amdgcn_s_setprio(0);
    // Compute phase.
    pp_multiply<C, Tag>(acc, f);
    if (group == 0) pp_wait_vm<0>();  // B of slice s+1, read from the next phase on
    pp_barrier();
    h = h >= 3 ? h - 3 : h + 2;
  }
  if (group == 0) pp_barrier();  // matches group 1's idle phase: same barrier count
}

// MASK: edge tiles (M, N, K need not be multiples of the tile) for 16-bit
// operands whose contiguous dimension is a multiple of 8: loads past the
// operand read zeros and the epilogue stores only inside M x N.
template <class Tag, int EPI, bool AMN, bool BMN, bool MASK = false>
__global__ void __launch_bounds__(PingPongCfg::THREADS) gemm_mfma_pingpong_kernel(const GemmArgs p) {
  using C = PingPongCfgT<AMN ? 32 : 16>;  // the atom: see the notes at the top
  using At = typename C::At;
  using acc_t = typename At::acc_t;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: no divergent barriers
  const int group = wave >> 2;
  const int wm = group, wn = wave & 3;

  // One tile: its loads, K loop and epilogue.
  auto tile = [&](int t, int ln) {
    int tm, tn;
    schedule_tile(t, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * C::BM;
    const int n0 = tn * C::BN;

    PingPongPipe<AMN, BMN, C::At::M, MASK> pipe;
    pipe.init(p, smem, m0, n0, group, wave, ln, wm, wn);

    acc_t acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int v = 0; v < At::NACC; ++v) acc[i][j][v] = 0.0f;

    pp_mainloop<C, Tag, EPI, AMN, BMN, MASK>(acc, pipe, p.K, group);
    store_tile<C, EPI, MASK>(acc, p, m0 + wm * C::WTM, n0 + wn * C::WTN, ln);
  };
  if constexpr (MASK) {
    tile(blockIdx.x, lane);  // edge tiles: one tile per workgroup
  } else {
    // Whole tiles t = blockIdx.x, + gridDim.x, ...: one per workgroup when
    // the grid has a workgroup per tile; with a grid of one workgroup per CU
    // each workgroup walks its tiles in turn, so the next tile's first loads
    // are requested right after this tile's D stores are issued instead of
    // after they drain (a multiple of 8 workgroups keeps every tile on the
    // XCD the scheduler's order assigns it).
    const int ntiles = p.tiles_m * p.tiles_n;
    for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
      // The lane index, opaque to loop-invariant code motion: what depends
      // on it is formed inside each tile's iteration, not held in registers
      // across the K loop.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      tile(t, ln);
    }
  }
}

}  // namespace dgt
