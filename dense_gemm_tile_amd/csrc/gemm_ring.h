// The ring design of the 128x128 direct-to-LDS kernel
// (gemm_mfma_ring128.hip), written for a square tile of side ROWS.
//
// Same contraction and atom nest as the other matrix-core kernels (TVM TIRx
// `gemm`: "Algorithm" steps 1-3), with asynchronous operand staging in the
// spirit of Phobos `@pipeline`, laid out for CDNA4:
//
//  * 4 waves (2 x 2) per K group; each wave computes a (ROWS/2)x(ROWS/2)
//    block of the tile with v_mfma_f32_32x32x16 atoms. At ROWS = 128 that is
//    64 accumulator registers per lane and 80 KiB of LDS, so two workgroups
//    share a CU (or, with two K groups, one workgroup of 8 waves uses the
//    whole 160 KiB).
//  * LDS is a ring of five half-slots, each one operand of one K slice of
//    64; A of slice t lives in slot 2t % 5 and B in slot (2t+1) % 5.
//    Iteration s multiplies slice s; right after its barrier the slots of
//    slice s-1 are free and take B of slice s+1 and A of slice s+2, so every
//    load has one or two iterations to land.
//  * Operands are read in the layout they are stored in: a K-contiguous
//    operand (A stored [M][K], B stored [N][K]) fills a slot as ROWS rows of
//    128 bytes with chunk c of row r at c ^ ((r ^ r>>3) & 7), one
//    ds_read_b128 per fragment; an M/N-contiguous one (A stored [K][M], B
//    stored [K][N]) as 64 K-rows of 2*ROWS bytes with chunk c of row r at
//    c ^ (4 (r & 3)), two ds_read_b64_tr_b16 (transposed reads) per fragment.
//    No operand is transposed in registers.
//  * Staging, per operand and per call: direct, when the operand's base and
//    row pitch are multiples of 16 bytes and every edge that cuts its
//    contiguous dimension falls on a multiple of 8 elements: each lane's
//    buffer_load_dwordx4 writes its 16 bytes straight into LDS, and pieces
//    wholly outside the operand get an out-of-range offset, which the
//    hardware answers with zeros. Otherwise staged: the same 16-byte pieces
//    go through registers (read as the dword-aligned dwords that cover them
//    and shifted into place, so any 2-byte alignment works; the buffer's
//    record count ends at the dword holding the operand's last element),
//    elements past an edge are zeroed, and one ds_write_b128 per piece puts
//    them where the direct load would have.
//  * Edge tiles store D element by element with bounds checks; interior
//    tiles with 16-byte accesses.
#pragma once

#include "gemm_mfma_pingpong.h"

#include <type_traits>

namespace dgt {

template <int ROWS>
struct RingCfg {
  static constexpr int BM = ROWS, BN = ROWS, BK = 64;
  static constexpr int WM = 2, WN = 2, THREADS = WM * WN * 64;
  using At = Atom<32>;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / At::M, TN = WTN / At::N;
  static constexpr int KSTEPS = BK / At::K;
  static constexpr int HALF_BYTES = ROWS * BK * 2;  // one operand of one slice
  static constexpr int SLOTS = 5;
  static constexpr int LDS_BYTES = SLOTS * HALF_BYTES;
  static constexpr int LOADS = HALF_BYTES / 1024 / (THREADS / 64);  // per wave per half
  static constexpr int MIN_WG = (160 * 1024) / LDS_BYTES;  // workgroups per CU (KG = 1)
  // Only the 128x128 tile is built: a 256x256 four-wave form (128x128 per
  // wave) measured 23 % slower at 8192^3 than the two-group kernel.
  static_assert(ROWS == 128, "tile side 128");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
};
using Ring128Cfg = RingCfg<128>;

// Zero the 16-bit elements of a 16-byte piece from index nv (0..8) on.
__device__ inline u32x4 keep_first(u32x4 v, int nv) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const unsigned lo = 2 * d < nv ? 0x0000FFFFu : 0u;
    const unsigned hi = 2 * d + 1 < nv ? 0xFFFF0000u : 0u;
    v[d] &= lo | hi;
  }
  return v;
}

// Registers of one operand's staged pieces between their loads and their
// LDS writes: 16-bit values as the dwords that cover each piece (v, one more
// dword e) and the piece's byte shift sh; float32 values as two 16-byte
// halves (v, v2), rounded when written.
template <bool SRC32, int L>
struct RingStaged {
  u32x4 v[L];
  unsigned e[L], sh[L];
};
template <int L>
struct RingStaged<true, L> {
  u32x4 v[L], v2[L];
};

// One operand: its loads into a half-slot (direct or staged through
// registers) and its fragment reads. MN: stored with M (or N) contiguous.
// SRC32: the operand holds float32 values, staged only, each piece rounded
// to the kernel's 16-bit type (ties to even) on its way into LDS, where it
// takes the place a 16-bit piece would.
// Instruction i (0..3) of wave w writes LDS bytes [(4w + i) KiB, +1 KiB) of
// the half-slot, lane l the 16 bytes at l * 16 of that.
template <bool MN, int ROWS, bool SRC32 = false>
struct RingOperand {
  using Cfg = RingCfg<ROWS>;
  static constexpr int LOADS = Cfg::LOADS;
  static constexpr int NFRAG = Cfg::TM;   // atoms per wave along this operand
  static constexpr int RB = ROWS * 2;     // bytes of one K-row of an M/N-contiguous slot
  static constexpr int ESZ = SRC32 ? 4 : 2;  // bytes per stored element
  using Staged = RingStaged<SRC32, LOADS>;
  const char* X;  // operand base
  int64_t ld2;    // row pitch in bytes
  int64_t ext;    // bytes of the stored extent ((rows - 1) * ld + cols) * ESZ
  int r0;         // tile origin along M (or N)
  int rlim;       // M (or N)
  int klim;       // K
  int off[NFRAG];  // fragment read offsets of this lane's atoms, sub-step 0

  // Logical position of the piece lane `lane` moves in instruction i of wave
  // w: K-contiguous: tile row rr (0..ROWS-1) and K chunk cc (0..7) of the
  // slice (an instruction covers 8 rows of 128 bytes); M/N-contiguous: slice
  // K-row rr (0..63) and M/N chunk cc (0..ROWS/8-1) (an instruction covers
  // 1024/RB K-rows of RB bytes).
  __device__ static inline void piece(int w, int i, int lane, int& rr, int& cc) {
    if constexpr (!MN) {
      rr = (ROWS / 4) * w + 8 * i + (lane >> 3);
      cc = (lane & 7) ^ ((rr ^ (rr >> 3)) & 7);
    } else {
      constexpr int CPR = ROWS / 8;  // 16-byte chunks per K-row
      rr = 16 * w + (64 / CPR) * i + lane / CPR;
      cc = (lane % CPR) ^ (4 * (rr & 3));
    }
  }

  __device__ inline void init(const void* Xv, int64_t ld, int r0_, int rlim_, int klim_,
                              int wsub, int lane) {
    X = static_cast<const char*>(Xv);
    ld2 = ld * ESZ;
    r0 = r0_;
    rlim = rlim_;
    klim = klim_;
    ext = MN ? ((int64_t)(klim - 1) * ld + rlim) * ESZ : ((int64_t)(rlim - 1) * ld + klim) * ESZ;
    if constexpr (!MN) {
#pragma unroll
      for (int t = 0; t < NFRAG; ++t)
        off[t] = lds_off(wsub * (ROWS / 2) + t * 32 + (lane & 31), lane >> 5);
    } else {
      // Lane l (16-lane group g = l/16, s = l%16) of the first transposed
      // read names K-row 8 (l/32) + s/4 and columns 16 (g & 1) + 4 (s % 4)
      // .. +3 of its atom; the second read is 4 rows down, sub-step ks is 16
      // ks rows down (both keep r & 3, so the swizzle is unchanged).
      const int r = 8 * (lane >> 5) + ((lane & 15) >> 2);
#pragma unroll
      for (int t = 0; t < NFRAG; ++t) {
        const int col = wsub * (ROWS / 2) + t * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        off[t] = r * RB + (((col >> 3) ^ (4 * (r & 3))) << 4) + ((col & 7) << 1);
      }
    }
  }

  // Resource base and record count for slice t, and the byte offset of the
  // piece (rr, cc) from that base, or kOutOfRange if the piece lies wholly
  // outside the operand. `start` is the piece's first index along the
  // contiguous dimension and `lim` that dimension's size (for masking).
  __device__ inline const char* slice_base(int t) const {
    return MN ? X + (int64_t)t * Cfg::BK * ld2 + (int64_t)r0 * ESZ : X + (int64_t)r0 * ld2;
  }
  __device__ inline int piece_off(int t, int rr, int cc, int& start, int& lim) const {
    if constexpr (!MN) {
      start = t * Cfg::BK + cc * 8;
      lim = klim;
      const bool in = r0 + rr < rlim && start < klim;
      return in ? (int)(rr * ld2) + start * ESZ : kOutOfRange;
    } else {
      start = r0 + cc * 8;
      lim = rlim;
      const bool in = t * Cfg::BK + rr < klim && start < rlim;
      return in ? (int)(rr * ld2) + cc * 8 * ESZ : kOutOfRange;
    }
  }

  __device__ __forceinline__ void issue_direct(char* slot, int t, int w, int lane) const {
    static_assert(!SRC32, "float32 operands are staged");
    const char* b = slice_base(t);
    const auto rs = make_rsrc_n(b, nrec_from(X, ext, b));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      int rr, cc, start, lim;
      piece(w, i, lane, rr, cc);
      const int voff = piece_off(t, rr, cc, start, lim);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (pp_lds_ptr_t)(slot + (4 * w + i) * 1024), 16,
                                               voff, 0, 0, 0);
    }
  }

  // Staged loads of slice t: each 16-byte piece (2-byte aligned) is read as
  // the dwords that cover it, with dword-aligned addresses only: four from
  // the dword at or below its start and one more after them. The record
  // count then cuts at a dword boundary (the extent rounded up to a dword),
  // so no dword that holds part of an element is dropped and nothing past
  // the operand's last dword is read.
  __device__ __forceinline__ void load_staged(Staged& r, int t, int w, int lane) const {
    if constexpr (SRC32) {
      // Float32 elements are dword-aligned: each piece is two 16-byte loads
      // at its own address (out-of-range offsets read zeros).
      const char* b = slice_base(t);
      const auto rs = make_rsrc_n(b, nrec_from(X, ext, b));
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        int rr, cc, start, lim;
        piece(w, i, lane, rr, cc);
        const int off = piece_off(t, rr, cc, start, lim);
        r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        r.v2[i] = __builtin_amdgcn_raw_buffer_load_b128(
            rs, off == kOutOfRange ? kOutOfRange : off + 16, 0, 0);
      }
      return;
    } else {
    u32x4 (&v)[LOADS] = r.v;
    unsigned (&e)[LOADS] = r.e;
    unsigned (&sh)[LOADS] = r.sh;
    // The resource starts at the dword holding the slice's first byte, so
    // every dword-aligned offset below a piece's start is still >= 0.
    const char* b0 = slice_base(t);
    const int bshift = (int)((uintptr_t)b0 & 3);  // 0 or 2
    const char* b = b0 - bshift;
    const auto rs = make_rsrc_n(b, nrec_from(X, ext, b));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      int rr, cc, start, lim;
      piece(w, i, lane, rr, cc);
      const int off = piece_off(t, rr, cc, start, lim);
      // the piece's byte offset from the aligned base, and its position
      // within its first dword
      const int rel = off == kOutOfRange ? 0 : off + bshift;
      sh[i] = (unsigned)(rel & 3);
      const int aoff = off == kOutOfRange ? kOutOfRange : rel - (rel & 3);
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, aoff, 0, 0);
      e[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, aoff == kOutOfRange ? kOutOfRange : aoff + 16,
                                                  0, 0);
    }
    }
  }

  // Shift each piece into place (the dwords were read from the dword at or
  // below its start), zero the elements past the edge of the contiguous
  // dimension (pieces that straddle it), then write the pieces where a
  // direct load would have.
  // mode (float32 operands): 1 rounds to f16, 2 to bf16.
  __device__ __forceinline__ void store_staged(char* slot, const Staged& r, int t, int w, int lane,
                                               bool edge, int mode) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      u32x4 x;
      if constexpr (SRC32) {
        const f32x4 lo = __builtin_bit_cast(f32x4, r.v[i]);
        const f32x4 hi = __builtin_bit_cast(f32x4, r.v2[i]);
        const float f[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        x = round8_f32_16(f, mode);
      } else {
        x[0] = __builtin_amdgcn_alignbyte(r.v[i][1], r.v[i][0], r.sh[i]);
        x[1] = __builtin_amdgcn_alignbyte(r.v[i][2], r.v[i][1], r.sh[i]);
        x[2] = __builtin_amdgcn_alignbyte(r.v[i][3], r.v[i][2], r.sh[i]);
        x[3] = __builtin_amdgcn_alignbyte(r.e[i], r.v[i][3], r.sh[i]);
      }
      if (edge) {
        int rr, cc, start, lim;
        piece(w, i, lane, rr, cc);
        (void)piece_off(t, rr, cc, start, lim);
        x = keep_first(x, lim - start < 8 ? (lim - start > 0 ? lim - start : 0) : 8);
      }
      *reinterpret_cast<u32x4*>(slot + (4 * w + i) * 1024 + lane * 16) = x;
    }
  }

  __device__ __forceinline__ u32x4 read(const char* slot, int t, int ks) const {
    return read_at(slot, off[t], ks);
  }
  // The fragment whose sub-step-0 offset is o (one of off[]).
  __device__ __forceinline__ static u32x4 read_at(const char* slot, int o, int ks) {
    if constexpr (!MN) {
      return *reinterpret_cast<const u32x4*>(slot + (o ^ (ks << 5)));
    } else {
      typedef __attribute__((address_space(3))) pp_i16x4 lds_i16x4;
      const char* q = slot + o + ks * 16 * RB;
      const pp_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q));
      const pp_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 4 * RB));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{l2.x, l2.y, h2.x, h2.y};
    }
  }
};

// The epilogue of one atom row of a wave's 64x64 block (after the K groups'
// exchange each group finishes one of the two rows).
template <class C>
struct RingRow : C {
  static constexpr int TM = 1;
};

// Rows past the last whole tile row (at most kMaxFold: p.mfold) folded into
// that tile row's workgroups, so that a shape such as 4097 x 1000 runs as
// 256 tiles (one per CU) instead of 264. The extra rows form one row of
// 16x16x32 atoms under the tile: wave w of each K group owns the 32
// columns [32w, 32w+32) (two atoms). Their A values are loaded one slice
// ahead and before the slice's other loads, so every wait that covers those
// loads covers them too: for each extra row, lanes 0-31 load the slice's 64
// K values as 32 pairs (two 2-byte loads per lane, any alignment, rows past
// M and K past the end reading zeros), and each lane then gathers its
// fragment's four pairs with ds_bpermute. Lanes whose fragment row is not an
// extra row keep whatever they gather: their output rows are not stored.
// Their B fragments are read from the B slot the tile already holds. The K
// groups' sums meet through LDS after the loop, in group order, like the
// tile's.
constexpr int kMaxFold = 4;
struct RingFoldRow {  // the epilogue's view: one row of two 16x16 atoms
  using At = Atom<16>;
  static constexpr int TM = 1, TN = 2;
};

template <bool MN, int ROWS>
struct RingFold {
  using A16 = Atom<16>;
  // Slice t's A values of extra row i (row0 + i, i < nrows): lane l < 32
  // gets K values t*64 + 2l and +1 as one dword (zeros past M or K).
  __device__ static inline void load_pairs(unsigned (&pr)[kMaxFold], const uint16_t* A,
                                           int64_t lda, int row0, int nrows, int M, int K, int t,
                                           int lane) {
#pragma unroll
    for (int i = 0; i < kMaxFold; ++i) {
      const int row = row0 + i;
      const int k = t * 64 + 2 * lane;
      unsigned lo = 0u, hi = 0u;
      if (i < nrows && lane < 32 && row < M) {
        if (k < K) lo = MN ? A[(int64_t)k * lda + row] : A[(int64_t)row * lda + k];
        if (k + 1 < K) hi = MN ? A[(int64_t)(k + 1) * lda + row] : A[(int64_t)row * lda + k + 1];
      }
      pr[i] = lo | (hi << 16);
    }
  }
  // The A fragment of sub-step ks from the pairs: lane l (fragment row
  // l%16, K values 32 ks + 8 (l/16) .. +7) takes pairs 16 ks + 4 (l/16) .. +3
  // of extra row l%16.
  __device__ static inline u32x4 gather(const unsigned (&pr)[kMaxFold], int nrows, int ks,
                                        int lane) {
    const int src = 16 * ks + 4 * (lane >> 4);
    u32x4 f = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kMaxFold; ++i) {
      if (i < nrows) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const unsigned v = (unsigned)__builtin_amdgcn_ds_bpermute(4 * (src + d), (int)pr[i]);
          if ((lane & 15) == i) f[d] = v;
        }
      }
    }
    return f;
  }
  // B fragment of a 16x16x32 atom whose first column is col0 (within the
  // tile), sub-step ks, from a B slot in the ring's layout.
  __device__ static inline u32x4 read_b(const char* slot, int col0, int ks, int lane) {
    if constexpr (!MN) {
      // K-contiguous slot: row n, chunk 4 ks + l/16
      return *reinterpret_cast<const u32x4*>(slot + lds_off(col0 + (lane & 15), 4 * ks + (lane >> 4)));
    } else {
      // M/N-contiguous slot: two transposed reads give lane l column
      // col0 + l%16 at K rows 32 ks + 8 (l/16) .. +7; lane s of each group
      // of 16 names row 32 ks + 8 g + s/4, columns col0 + 4 (s%4) .. +3.
      typedef __attribute__((address_space(3))) pp_i16x4 lds_i16x4;
      constexpr int RB = ROWS * 2;
      const int s = lane & 15, g = lane >> 4;
      const int col = col0 + 4 * (s & 3);
      const int r = 32 * ks + 8 * g + (s >> 2);
      const char* q = slot + r * RB + (((col >> 3) ^ (4 * (r & 3))) << 4) + ((col & 7) << 1);
      const pp_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q));
      const pp_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 4 * RB));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{l2.x, l2.y, h2.x, h2.y};
    }
  }
};

// KG K groups of 4 waves each: group g multiplies the tile's slices g, g+KG,
// g+2KG, ... with a ring of its own; with KG = 2 a tile takes 160 KiB of LDS
// and 8 waves, so grids of about one tile per CU still give every SIMD two
// independent waves. The groups' accumulators are summed in group order.
// ROWS: tile side (128: 64x64 per wave, two workgroups per CU with KG = 1).
// STAGING: operands staged through registers are supported (otherwise both
// must be direct). SRC32: both operands hold float32 values (staged, rounded
// to Tag's type with mode p.src32).
// FOLD: the instantiation for p.mfold > 0 (two K groups, 16-bit operands),
// which leaves out the early C requests to make room for the folded rows.
// STG2: exactly one operand staged (16-bit values; which one is uniform at
// run time): its loads are requested three slices ahead into two register
// sets taken in turn, instead of two slices ahead into one, so each staged
// load has two iterations to land instead of one.
template <int ROWS, class Tag, int EPI, bool AMN, bool BMN, int KG, bool STAGING, bool SRC32 = false,
          bool FOLD = false, bool STG2 = false>
__global__ void __launch_bounds__(RingCfg<ROWS>::THREADS * KG, RingCfg<ROWS>::MIN_WG / KG)
gemm_ring_kernel(const GemmArgs p) {
  using C = RingCfg<ROWS>;
  using At = typename C::At;
  using acc_t = typename At::acc_t;
  __shared__ __attribute__((aligned(1024))) char lds[KG * C::LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;  // K group
  const int w = wave & 3;     // wave within its group
  const int wm = w >> 1, wn = w & 1;
  char* const smem = lds + grp * C::LDS_BYTES;
  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  static_assert(!SRC32 || STAGING, "float32 operands are staged");
  RingOperand<AMN, ROWS, SRC32> a;
  RingOperand<BMN, ROWS, SRC32> b;
  a.init(p.A, p.lda, m0, p.M, p.K, wm, lane);
  b.init(p.B, p.ldb, n0, p.N, p.K, wn, lane);
  const int mode = p.src32;
  // Staging modes (uniform over the launch) and, for staged operands, whether
  // this tile's pieces can straddle the edge of the contiguous dimension.
  const bool a_dir = !SRC32 && (!STAGING || p.a_direct);
  const bool b_dir = !SRC32 && (!STAGING || p.b_direct);
  const bool a_edge = AMN ? (m0 + C::BM > p.M && p.M % 8 != 0) : (p.K % 8 != 0);
  const bool b_edge = BMN ? (n0 + C::BN > p.N && p.N % 8 != 0) : (p.K % 8 != 0);
  const bool staged = !a_dir || !b_dir;
  // Atoms of this wave that hold outputs inside M x N (uniform per wave): on
  // edge tiles the others are neither read nor multiplied.
  auto nvalid = [](int lo, int lim, int n) {
    const int v = (lim - lo + 31) / 32;
    return v < 0 ? 0 : (v > n ? n : v);
  };
  const int nvi = nvalid(m0 + wm * C::WTM, p.M, C::TM);
  const int nvj = nvalid(n0 + wn * C::WTN, p.N, C::TN);
  const bool full_wave = nvi == C::TM && nvj == C::TN;
  // Folded rows (see RingFold).
  static_assert(!FOLD || (KG == 2 && !SRC32), "rows are folded with two K groups, 16-bit operands");
  using A16 = Atom<16>;
  const bool fold = FOLD && tm == p.tiles_m - 1;  // uniform
  const int frow0 = m0 + C::BM, fnrows = p.mfold;
  typename A16::acc_t facc[1][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int v = 0; v < A16::NACC; ++v) facc[0][t][v] = 0.0f;
  unsigned fpc[kMaxFold], fpn[kMaxFold];  // folded rows' A pairs: this slice, the next

  acc_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) acc[i][j][v] = 0.0f;

  // This group's slices: local index j is the tile's slice j*KG + grp.
  const int KT = (p.K + C::BK - 1) / C::BK;
  const int JT = (KT + KG - 1) / KG;                  // iterations (all groups)
  const int NJ = KT > grp ? (KT - grp + KG - 1) / KG : 0;  // this group's slices
  auto gs = [&](int j) { return j * KG + grp; };
  auto slot = [&](int h) { return smem + (h % C::SLOTS) * C::HALF_BYTES; };
  // Staged operands' pieces between their loads and their LDS writes.
  typename RingOperand<AMN, ROWS, SRC32>::Staged ra;
  typename RingOperand<BMN, ROWS, SRC32>::Staged rb;

  // With two K groups each group finishes one atom row of its waves' blocks
  // (row grp). On interior tiles that read C it requests those C values
  // right after the prologue's loads, so they arrive while the K loop runs
  // instead of after it (32 registers per lane).
  constexpr bool PRE_C = KG == 2 && EPI != EPI_BETA0 && !FOLD && !STG2;
  const bool inner = m0 + C::BM <= p.M && n0 + C::BN <= p.N;
  const bool pre_c = PRE_C && p.wide_epi && inner;
  WideC<RingRow<C>> cpre;

  // Multiply local slice j (edge waves: only their atoms that hold outputs
  // inside M x N; the branch is uniform per wave), and the folded rows.
  auto multiply = [&](int j) {
    const char* sa = slot(2 * j);
    const char* sb = slot(2 * j + 1);
  #pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      u32x4 fa[C::TM], fb[C::TN];
  #pragma unroll
      for (int i = 0; i < C::TM; ++i) fa[i] = a.read(sa, i, ks);
  #pragma unroll
      for (int jj = 0; jj < C::TN; ++jj) fb[jj] = b.read(sb, jj, ks);
  #pragma unroll
      for (int i = 0; i < C::TM; ++i)
  #pragma unroll
        for (int jj = 0; jj < C::TN; ++jj)
          if (full_wave || (i < nvi && jj < nvj))
            acc[i][jj] = At::mma(Tag{}, fa[i], fb[jj], acc[i][jj]);
    }
    if constexpr (FOLD) {
      if (fold) {
  #pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u32x4 fa16 = RingFold<AMN, ROWS>::gather(fpc, fnrows, ks, lane);
  #pragma unroll
          for (int t = 0; t < 2; ++t)
            facc[0][t] = A16::mma(Tag{}, fa16,
                                  RingFold<BMN, ROWS>::read_b(sb, 32 * w + 16 * t, ks, lane),
                                  facc[0][t]);
        }
      }
    }
  };

  if constexpr (STG2) {
    static_assert(STAGING && !SRC32, "two-deep staging takes 16-bit values");
    // X: the staged operand (A when !a_dir, else B); X of local slice s sits
    // in register set s % 2 from its request (three slices ahead) until its
    // LDS write (one slice ahead).
    using Stg = typename RingOperand<AMN, ROWS, false>::Staged;
    static_assert(std::is_same<Stg, typename RingOperand<BMN, ROWS, false>::Staged>::value,
                  "both operands stage through the same register set type");
    Stg st0, st1;
    const bool xa = !a_dir;
    auto x_load = [&](Stg& r, int j) {
      if (xa) a.load_staged(r, gs(j), w, lane);
      else b.load_staged(r, gs(j), w, lane);
    };
    auto x_store = [&](const Stg& r, int j) {
      if (xa) a.store_staged(slot(2 * j), r, gs(j), w, lane, a_edge, 0);
      else b.store_staged(slot(2 * j + 1), r, gs(j), w, lane, b_edge, 0);
    };
    if constexpr (FOLD) {
      if (fold && NJ > 0)
        RingFold<AMN, ROWS>::load_pairs(fpc, static_cast<const uint16_t*>(p.A), p.lda, frow0,
                                        fnrows, p.M, p.K, gs(0), lane);
    }
    if (NJ > 0) {
      if (xa) {
        x_load(st0, 0);
        if constexpr (!SRC32) b.issue_direct(slot(1), gs(0), w, lane);
      } else {
        if constexpr (!SRC32) a.issue_direct(slot(0), gs(0), w, lane);
        x_load(st0, 0);
        if constexpr (!SRC32) { if (NJ > 1) a.issue_direct(slot(2), gs(1), w, lane); }
      }
      pp_wait_vm<0>();
      x_store(st0, 0);
      if (NJ > 1) x_load(st1, 1);
      if (NJ > 2) x_load(st0, 2);
      // X of local slice 1 is written in iteration 0; slice 2 may stay in flight.
      if (NJ > 2) pp_wait_vm_lgkm0<2 * C::LOADS>();
      else pp_wait_vm_lgkm0<0>();
    }
    pp_barrier();
    // Iteration j writes X of local slice j+1 from `sx` and requests X of
    // j+3 into the same set; the direct operand's loads are as in the
    // one-deep loop. At its end every load but the newest requests (X of
    // j+3, and a direct A of j+2) has landed: the slice read next and X of
    // j+2, which the next iteration writes.
    auto iter = [&](int j, Stg& sx) {
      if (j < NJ) {
        if constexpr (FOLD) {
          if (fold && j + 1 < NJ)
            RingFold<AMN, ROWS>::load_pairs(fpn, static_cast<const uint16_t*>(p.A), p.lda, frow0,
                                            fnrows, p.M, p.K, gs(j + 1), lane);
        }
        if (j + 1 < NJ) x_store(sx, j + 1);
        if constexpr (!SRC32) {
          if (xa) {
            if (j + 1 < NJ) b.issue_direct(slot(2 * j + 3), gs(j + 1), w, lane);
          } else {
            if (j + 2 < NJ) a.issue_direct(slot(2 * j + 4), gs(j + 2), w, lane);
          }
        }
        if (j + 3 < NJ) x_load(sx, j + 3);
        multiply(j);
        if (xa) {
          if (j + 3 < NJ) pp_wait_vm_lgkm0<2 * C::LOADS>();
          else pp_wait_vm_lgkm0<0>();
        } else {
          if (j + 3 < NJ) pp_wait_vm_lgkm0<3 * C::LOADS>();
          else if (j + 2 < NJ) pp_wait_vm_lgkm0<C::LOADS>();
          else pp_wait_vm_lgkm0<0>();
        }
      }
      pp_barrier();
      if constexpr (FOLD) {
        if (fold) {
#pragma unroll
          for (int i = 0; i < kMaxFold; ++i) fpc[i] = fpn[i];
        }
      }
    };
    for (int j = 0; j < JT; j += 2) {
      iter(j, st1);
      if (j + 1 < JT) iter(j + 1, st0);
    }
  } else {
    // Prologue: local slice 0 into slots 0 and 1, then A of local slice 1
    // (direct) into slot 2, or local slice 1 (staged) into registers. The
    // folded rows' A of slice 0 goes first.
    if constexpr (FOLD) {
      if (fold && NJ > 0)
        RingFold<AMN, ROWS>::load_pairs(fpc, static_cast<const uint16_t*>(p.A), p.lda, frow0,
                                        fnrows, p.M, p.K, gs(0), lane);
    }
    if (NJ > 0) {
      if (a_dir) {
        if constexpr (!SRC32) a.issue_direct(slot(0), gs(0), w, lane);
      } else {
        a.load_staged(ra, gs(0), w, lane);
      }
      if (b_dir) {
        if constexpr (!SRC32) b.issue_direct(slot(1), gs(0), w, lane);
      } else {
        b.load_staged(rb, gs(0), w, lane);
      }
      if constexpr (!SRC32) { if (a_dir && NJ > 1) a.issue_direct(slot(2), gs(1), w, lane); }
    }
    if constexpr (PRE_C) {
      if (pre_c)
        load_wide_c<RingRow<C>>(cpre, p, m0 + wm * C::WTM + grp * At::M, n0 + wn * C::WTN, lane);
    }
    constexpr int NC = PRE_C ? C::TN * At::NACC / 4 : 0;  // C loads per lane
    if (NJ > 0) {
      if (staged) {
        pp_wait_vm<0>();
        if (!a_dir) a.store_staged(slot(0), ra, gs(0), w, lane, a_edge, mode);
        if (!b_dir) b.store_staged(slot(1), rb, gs(0), w, lane, b_edge, mode);
        if (NJ > 1) {
          if (!a_dir) a.load_staged(ra, gs(1), w, lane);
          if (!b_dir) b.load_staged(rb, gs(1), w, lane);
        }
        pp_wait_lgkm0();
      } else if (NJ > 1) {
        // A of local slice 1 (and the C requests) may stay in flight
        if (pre_c) pp_wait_vm_lgkm0<C::LOADS + NC>();
        else pp_wait_vm_lgkm0<C::LOADS>();
      } else {
        if (pre_c) pp_wait_vm_lgkm0<NC>();
        else pp_wait_vm_lgkm0<0>();
      }
    }
    pp_barrier();

    for (int j = 0; j < JT; ++j) {
      if (j < NJ) {
        // Folded rows: A of local slice j+1, before this iteration's other
        // loads.
        if constexpr (FOLD) {
          if (fold && j + 1 < NJ)
            RingFold<AMN, ROWS>::load_pairs(fpn, static_cast<const uint16_t*>(p.A), p.lda, frow0,
                                            fnrows, p.M, p.K, gs(j + 1), lane);
        }
        // Staged operands: local slice j+1 arrived in registers during the
        // previous iteration (this waits for every older load); write it into
        // its slots (A: 2j+2, left by B of j-2; B: 2j+3, left by A of j-1),
        // then request local slice j+2 into the same registers.
        if (staged && j + 1 < NJ) {
          pp_wait_vm<0>();
          if (!a_dir) a.store_staged(slot(2 * j + 2), ra, gs(j + 1), w, lane, a_edge, mode);
          if (!b_dir) b.store_staged(slot(2 * j + 3), rb, gs(j + 1), w, lane, b_edge, mode);
        }
        // Direct loads into the slots local slice j-1 has left: B of j+1
        // first, then A of j+2 (slot 2j+4, left by B of j-1).
        if constexpr (!SRC32) {
          if (b_dir && j + 1 < NJ) b.issue_direct(slot(2 * j + 3), gs(j + 1), w, lane);
          if (a_dir && j + 2 < NJ) a.issue_direct(slot(2 * j + 4), gs(j + 2), w, lane);
        }
        if (staged && j + 2 < NJ) {
          if (!a_dir) a.load_staged(ra, gs(j + 2), w, lane);
          if (!b_dir) b.load_staged(rb, gs(j + 2), w, lane);
        }

        multiply(j);

        // Local slice j+1 must be in LDS by the next barrier. A direct B of
        // j+1 was issued first in this iteration, so at most the one
        // half-slice request that followed it (A of j+2: 4 direct loads or 8
        // staged ones) may stay in flight; a direct A of j+1 is older still.
        // Without a direct B, the staged wait at the top of this iteration
        // already covered every older load. LDS reads and staged writes must
        // be complete.
        if (b_dir) {
          if (j + 2 < NJ && a_dir) pp_wait_vm_lgkm0<C::LOADS>();
          else if (j + 2 < NJ) pp_wait_vm_lgkm0<2 * C::LOADS>();  // staged: two loads per piece
          else pp_wait_vm_lgkm0<0>();
        } else {
          pp_wait_lgkm0();
        }
      }
      pp_barrier();
      if constexpr (FOLD) {
        if (fold) {
#pragma unroll
          for (int i = 0; i < kMaxFold; ++i) fpc[i] = fpn[i];
        }
      }
    }
  }

  if constexpr (KG == 1) {
    if (inner) store_tile<C, EPI, false>(acc, p, m0 + wm * C::WTM, n0 + wn * C::WTN, lane);
    else store_tile<C, EPI, true>(acc, p, m0 + wm * C::WTM, n0 + wn * C::WTN, lane);
  } else {
    static_assert(KG == 2 && C::TM == 2, "two K groups, each finishing one atom row");
    // Group g hands atom row 1-g to the other group through LDS (every
    // group is past its last read of the ring: the loop ended on a
    // barrier), then finishes atom row g as (group 0's sum) + (group 1's).
    constexpr int NV = C::TN * At::NACC;  // registers of one atom row
    float* x = reinterpret_cast<float*>(lds);
    {
      float* dst = x + (grp * 4 + w) * NV * 64 + lane;
#pragma unroll
      for (int jj = 0; jj < C::TN; ++jj)
#pragma unroll
        for (int v = 0; v < At::NACC; ++v)  // (a select: no dynamic index into registers)
          dst[(jj * At::NACC + v) * 64] = grp == 0 ? acc[1][jj][v] : acc[0][jj][v];
    }
    // Folded rows: group 1 hands its sums to group 0 (after the 64 KiB the
    // tile's exchange uses).
    float* fx_lds = x + 8 * NV * 64;
    if constexpr (FOLD) {
      if (fold && grp == 1) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int v = 0; v < A16::NACC; ++v) fx_lds[(w * 8 + t * 4 + v) * 64 + lane] = facc[0][t][v];
      }
    }
    pp_wait_lgkm0();
    pp_barrier();
    acc_t fin[1][C::TN];
    {
      const float* src = x + ((1 - grp) * 4 + w) * NV * 64 + lane;
#pragma unroll
      for (int jj = 0; jj < C::TN; ++jj)
#pragma unroll
        for (int v = 0; v < At::NACC; ++v) {
          const float other = src[(jj * At::NACC + v) * 64];
          fin[0][jj][v] = grp == 0 ? acc[0][jj][v] + other : other + acc[1][jj][v];
        }
    }
    const int r0 = m0 + wm * C::WTM + grp * At::M;
    if (inner) store_tile<RingRow<C>, EPI, false>(fin, p, r0, n0 + wn * C::WTN, lane, cpre, pre_c);
    else store_tile<RingRow<C>, EPI, true>(fin, p, r0, n0 + wn * C::WTN, lane);
    if constexpr (FOLD) {
      if (fold && grp == 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int v = 0; v < A16::NACC; ++v) facc[0][t][v] += fx_lds[(w * 8 + t * 4 + v) * 64 + lane];
        store_tile<RingFoldRow, EPI, true>(facc, p, m0 + C::BM, n0 + 32 * w, lane);
      }
    }
  }
}

}  // namespace dgt
