// Matrix-core (MFMA) GEMM kernel for gfx950, templated on the tile
// configuration, the operand type, the stored orientation of A and B, and
// whether edge masking is compiled in.
//
// The design follows the steps both reference designs share -- tile the output,
// stage operand boxes through on-chip memory, feed fixed matrix-core atoms and
// accumulate in place over K, then run the alpha/beta epilogue once per tile
// (TVM TIRx `gemm`: "Algorithm" steps 1-3; Phobos `@tensorcore`: the gemm
// kernel pair and its `@pipeline` staging) -- laid out for CDNA4:
//
//  * one workgroup per output tile, chosen by an XCD-aware grouped scheduler;
//  * global -> VGPR -> LDS staging with 128-bit loads (buffer loads with a
//    scalar base per K step on unmasked tiles), two LDS stages over K, global
//    loads issued two K steps ahead, fragments read one K sub-step ahead, one
//    barrier per K step;
//  * LDS rows hold 64 K-values (128 bytes, eight 16-byte chunks) of one M (or
//    N) index; chunk c of row r lives at chunk position c ^ ((r ^ (r>>3)) & 7),
//    an XOR swizzle instead of row padding (the sm_80 Phobos variant keeps its
//    tiles at their declared size the same way);
//  * operands stored with M (or N) contiguous are transposed in registers
//    while staging, so every LDS tile is K-contiguous and each lane fetches its
//    8 consecutive K-values of one row with a single 128-bit LDS read;
//  * wave64 fragments for v_mfma_f32_32x32x16_{f16,bf16} and
//    v_mfma_f32_16x16x32_{f16,bf16}, accumulators kept in registers;
//  * masked edges: out-of-range A/B elements are staged as zeros (their
//    products are exactly zero), C loads and D stores are predicated.
#pragma once

#include "common.h"

namespace dgt {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct TagF16 {};
struct TagBF16 {};

// ---------------------------------------------------------------- atoms ----
// Per-lane ownership of one MFMA atom on a 64-lane wave.
//  A fragment: lane l holds 8 consecutive K-values of atom row frag_row(l),
//              starting at K offset 8*frag_koct(l).
//  B fragment: the same with atom column in place of atom row.
//  Accumulator element v of lane l is atom entry (acc_row(l,v), acc_col(l)).
// Any K order shared by A and B gives the same sum, so only the row/column
// ownership below has to match the hardware exactly.
template <int AM>
struct Atom;

template <>
struct Atom<32> {  // v_mfma_f32_32x32x16_*: 16 f32 accumulators per lane
  static constexpr int M = 32, N = 32, K = 16, NACC = 16;
  using acc_t = f32x16;
  __device__ static inline int frag_row(int l) { return l & 31; }
  __device__ static inline int frag_koct(int l) { return l >> 5; }
  __device__ static inline int acc_row(int l, int v) { return 8 * (v >> 2) + 4 * (l >> 5) + (v & 3); }
  __device__ static inline int acc_col(int l) { return l & 31; }
  __device__ static inline acc_t mma(TagF16, u32x4 a, u32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline acc_t mma(TagBF16, u32x4 a, u32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Atom<16> {  // v_mfma_f32_16x16x32_*: 4 f32 accumulators per lane
  static constexpr int M = 16, N = 16, K = 32, NACC = 4;
  using acc_t = f32x4;
  // v_mfma_f32_16x16x16_*: the same rows, columns and accumulator layout over
  // 16 K-values; lane l holds 4 consecutive K-values starting at 4*(l >> 4).
  __device__ static inline acc_t mma16(TagF16, u32x2 a, u32x2 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static inline acc_t mma16(TagBF16, u32x2 a, u32x2 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
  __device__ static inline int frag_row(int l) { return l & 15; }
  __device__ static inline int frag_koct(int l) { return l >> 4; }
  __device__ static inline int acc_row(int l, int v) { return 4 * (l >> 4) + v; }
  __device__ static inline int acc_col(int l) { return l & 15; }
  __device__ static inline acc_t mma(TagF16, u32x4 a, u32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline acc_t mma(TagBF16, u32x4 a, u32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// --------------------------------------------------------- configuration ----
// KG > 1 splits K over KG groups of WM x WN waves: group g takes K steps
// g, g + KG, g + 2KG, ... of the same output tile into its own pair of LDS
// stages, and the groups' accumulators are summed through LDS in group order
// at the end (a fixed order, so results do not vary from run to run).
template <int BM_, int BN_, int WM_, int WN_, int ATOM_, int KG_ = 1>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WM = WM_, WN = WN_, KG = KG_;
  static constexpr int GROUP_THREADS = WM * WN * 64;  // one K group
  static constexpr int THREADS = GROUP_THREADS * KG;
  using At = Atom<ATOM_>;
  static constexpr int WTM = BM / WM, WTN = BN / WN;     // one wave's sub-tile
  static constexpr int TM = WTM / At::M, TN = WTN / At::N;  // atoms per wave
  static constexpr int KSTEPS = BK / At::K;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int GROUP_LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int LDS_BYTES = KG * GROUP_LDS_BYTES;
  // Accumulators that groups 1..KG-1 hand to group 0 (f32, lane-major).
  static constexpr int XFER_BYTES = (KG - 1) * WM * WN * TM * TN * At::NACC * 64 * 4;
  // The masked kernel's interior-tile paths (whole-step unmasked loads, 16-byte
  // stores) are compiled in only where the accumulators leave registers for
  // both loaders: with 256 accumulators per lane they would spill.
  static constexpr bool INNER_PATHS = TM * TN * At::NACC <= 64;
  static_assert(WTM % At::M == 0 && WTN % At::N == 0, "wave tile must hold whole atoms");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
  static_assert(XFER_BYTES <= LDS_BYTES, "the K-group sum is staged in the operand LDS");
  static_assert(THREADS <= 1024, "at most 1024 threads per workgroup");
};

// Byte offset of 16-byte chunk `chunk` (0..7) of LDS row `row` (128 bytes).
__device__ static inline int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// --------------------------------------------------------------- staging ----
// A buffer resource over `base` (bytes), used by the unmasked loaders: the
// per-lane byte offset stays in one VGPR and the per-piece step is a scalar.
__device__ static inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF,
                                           0x00020000);
}

// Rounding of one float32 value to a 16-bit pattern, to nearest with ties to
// even: mode 1 gives f16 (the hardware conversion, which rounds so in the
// default mode), mode 2 bf16 (on the bit pattern; NaN stays a quiet NaN).
__device__ inline unsigned round_f32_16(float x, int mode) {
  if (mode == 1) return __builtin_bit_cast(unsigned short, (_Float16)x);
  const unsigned u = __builtin_bit_cast(unsigned, x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// Eight float32 values rounded and packed into one 16-byte piece.
__device__ inline u32x4 round8_f32_16(const float (&f)[8], int mode) {
  u32x4 r;
  r.x = round_f32_16(f[0], mode) | (round_f32_16(f[1], mode) << 16);
  r.y = round_f32_16(f[2], mode) | (round_f32_16(f[3], mode) << 16);
  r.z = round_f32_16(f[4], mode) | (round_f32_16(f[5], mode) << 16);
  r.w = round_f32_16(f[6], mode) | (round_f32_16(f[7], mode) << 16);
  return r;
}

// One operand's R x 64 box (R rows of M or N, 64 K-values) per K step.
// KCONTIG: element (r, k) is X[(r0 + r) * ld + k0 + k]  (A with transA = 0,
//          B with transB = 1); otherwise X[(k0 + k) * ld + r0 + r].
// Each thread moves NL 16-byte pieces: for KCONTIG, NL chunks of 8 K-values
// (piece i covers box row (tid >> 3) + i * THREADS / 8); otherwise one block of
// NL K-rows x 8 row-values, transposed in registers on the way to LDS.
template <int R, int THREADS, bool KCONTIG, bool MASK>
struct Stager {
  static constexpr int NL = R * 64 / (8 * THREADS);
  static_assert(NL == 2 || NL == 4 || NL == 8, "stager expects 2, 4 or 8 pieces per thread");
  static_assert(KCONTIG || (R / 8) * (64 / NL) == THREADS, "one block per thread");
  u32x4 v[NL];

  __device__ static inline u32x4 load_partial(const uint16_t* p, int n_valid) {
    uint16_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) e[q] = q < n_valid ? p[q] : (uint16_t)0;
    u32x4 r;
    r.x = e[0] | ((unsigned)e[1] << 16);
    r.y = e[2] | ((unsigned)e[3] << 16);
    r.z = e[4] | ((unsigned)e[5] << 16);
    r.w = e[6] | ((unsigned)e[7] << 16);
    return r;
  }

  // A whole piece of an operand whose rows are not 16-byte aligned (vw in
  // {4, 2, 1}): one 16-byte global load at the piece's own 2-byte-aligned
  // address, which this target serves unaligned, so nothing has to be packed
  // (and waited for) here.
  __device__ static inline u32x4 load_narrow(const uint16_t* p, int) {
    typedef u32x4 u32x4_a2 __attribute__((aligned(2)));
    return *reinterpret_cast<const u32x4_a2*>(p);
  }

  __device__ static inline unsigned round16(float x, int mode) { return round_f32_16(x, mode); }
  __device__ static inline u32x4 round8(const float (&f)[8], int mode) {
    return round8_f32_16(f, mode);
  }
  // n_valid (0..8) float32 values of a piece, vw-element loads when whole.
  __device__ static inline u32x4 load_f32(const float* q, int n_valid, int vw, int mode) {
    float f[8];
    if (n_valid == 8 && vw == 4) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(q);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(q + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = lo[e], f[e + 4] = hi[e];
    } else if (n_valid == 8 && vw == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 t = *reinterpret_cast<const float2*>(q + 2 * e);
        f[2 * e] = t.x;
        f[2 * e + 1] = t.y;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = e < n_valid ? q[e] : 0.0f;
    }
    return round8(f, mode);
  }

  // Issue the global loads of the box at (r0, k0). rlim / klim: number of
  // valid rows / K-values of the whole operand (used only when MASK). vw
  // (MASK only): the operand's staging vector width in elements; below 8
  // (16 bytes) its pieces are not 16-byte aligned and are read in narrower
  // loads. src32 (MASK only): 0 for 16-bit operands; 1 / 2 for float32
  // operands rounded to f16 / bf16 here. whole (MASK only, uniform over the
  // workgroup): the box lies inside the operand, so its pieces need no
  // bounds checks: a 16-byte-aligned operand takes the unmasked kernel's
  // buffer loads, a 16-bit operand with narrower rows one 16-byte global load
  // per piece; the masked kernel's interior tiles do so on every whole K step.
  // pieces (MASK only, uniform; the operand is 16-byte aligned, 16-bit, and
  // its offsets fit 32 bits): every piece of this box is wholly inside or
  // wholly outside the operand, so the buffer loads serve it too, with an
  // out-of-range offset for the outside pieces, which the hardware answers
  // with zeros.
  __device__ __forceinline__ void load(const void* __restrict__ Xv, int64_t ld, int r0, int rlim,
                                       int k0, int klim, int tid, int vw = 8, int src32 = 0,
                                       bool whole = false, bool pieces = false) {
    const uint16_t* __restrict__ X = static_cast<const uint16_t*>(Xv);
    const float* __restrict__ X32 = static_cast<const float*>(Xv);
    if (!MASK || (whole && vw == 8)) {
      if constexpr (KCONTIG) {
        const auto rs = make_rsrc(X + (int64_t)r0 * ld + k0);
        const int voff = (int)(((tid >> 3) * ld + ((tid & 7) << 3)) * 2);
        const int step = (int)((THREADS / 8) * ld * 2);
#pragma unroll
        for (int i = 0; i < NL; ++i)
          v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, i * step, 0);
      } else {
        const int rc = tid % (R / 8), kb = tid / (R / 8);
        const auto rs = make_rsrc(X + (int64_t)k0 * ld + r0);
        const int voff = (int)(((kb * NL) * ld + rc * 8) * 2);
        const int step = (int)(ld * 2);
#pragma unroll
        for (int j = 0; j < NL; ++j)
          v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, j * step, 0);
      }
    } else if (pieces) {
      // Offset 2^31: every dword of the 16-byte access lies at or past the
      // resource's 0x7FFFFFFF records, so nothing is read and zeros return.
      // Inside pieces stay below 2^31 - 4096 (the host's 32-bit offset rule).
      constexpr int kOut = (int)0x80000000u;
      if constexpr (KCONTIG) {
        const auto rs = make_rsrc(X + (int64_t)r0 * ld + k0);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int id = tid + i * THREADS;
          const int rr = id >> 3, kk = (id & 7) << 3;
          const bool in = r0 + rr < rlim && k0 + kk < klim;
          v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, in ? (int)((rr * ld + kk) * 2) : kOut,
                                                       0, 0);
        }
      } else {
        const int rc = tid % (R / 8), kb = tid / (R / 8);
        const auto rs = make_rsrc(X + (int64_t)k0 * ld + r0);
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int kk = kb * NL + j, rr = rc * 8;
          const bool in = k0 + kk < klim && r0 + rr < rlim;
          v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, in ? (int)((kk * ld + rr) * 2) : kOut,
                                                       0, 0);
        }
      }
    } else if (whole && !src32) {
      // Whole box of an operand whose rows are not 16-byte aligned: the same
      // pieces as 16-byte global loads at their own (2-byte aligned)
      // addresses, which this target serves unaligned (the compiler itself
      // merges eight 16-bit loads into one such load); no bounds checks.
      typedef u32x4 u32x4_a2 __attribute__((aligned(2)));
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        int64_t off;
        if constexpr (KCONTIG) {
          const int id = tid + i * THREADS;
          off = (int64_t)(r0 + (id >> 3)) * ld + k0 + ((id & 7) << 3);
        } else {
          off = (int64_t)(k0 + (tid / (R / 8)) * NL + i) * ld + r0 + (tid % (R / 8)) * 8;
        }
        v[i] = *reinterpret_cast<const u32x4_a2*>(X + off);
      }
    } else if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int id = tid + i * THREADS;
        const int r = r0 + (id >> 3);
        const int k = k0 + ((id & 7) << 3);
        const int64_t off = (int64_t)r * ld + k;
        const uint16_t* p = X + off;
        if (r < rlim && k < klim && src32) {
          v[i] = load_f32(X32 + off, klim - k < 8 ? klim - k : 8, vw, src32);
        } else if (r < rlim && k + 8 <= klim) {
          v[i] = vw == 8 ? *reinterpret_cast<const u32x4*>(p) : load_narrow(p, vw);
        } else if (r < rlim && k < klim) {
          v[i] = load_partial(p, klim - k < 8 ? klim - k : 8);
        } else {
          v[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    } else {
      const int rc = tid % (R / 8);
      const int kb = tid / (R / 8);
      const int r = r0 + rc * 8;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int k = k0 + kb * NL + j;
        const int64_t off = (int64_t)k * ld + r;
        const uint16_t* p = X + off;
        if (k < klim && r < rlim && src32) {
          v[j] = load_f32(X32 + off, rlim - r < 8 ? rlim - r : 8, vw, src32);
        } else if (k < klim && r + 8 <= rlim) {
          v[j] = vw == 8 ? *reinterpret_cast<const u32x4*>(p) : load_narrow(p, vw);
        } else if (k < klim && r < rlim) {
          v[j] = load_partial(p, rlim - r < 8 ? rlim - r : 8);
        } else {
          v[j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }

  // 16-bit element c (0..7) of a 16-byte piece, packed with a neighbour.
  __device__ static inline unsigned pack2(const u32x4& lo, const u32x4& hi, int c) {
    const unsigned a = lo[c >> 1], b = hi[c >> 1];
    return (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
  }

  __device__ inline void store(char* __restrict__ lds, int tid) const {
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int id = tid + i * THREADS;
        *reinterpret_cast<u32x4*>(lds + lds_off(id >> 3, id & 7)) = v[i];
      }
    } else {
      const int rc = tid % (R / 8);
      const int kb = tid / (R / 8);
      const int kofs = kb * NL;  // first K-value of this block within the box
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int row = rc * 8 + c;
        char* dst = lds + lds_off(row, kofs >> 3) + ((kofs & 7) << 1);
        if constexpr (NL == 8) {
          u32x4 o;
          o.x = pack2(v[0], v[1], c);
          o.y = pack2(v[2], v[3], c);
          o.z = pack2(v[4], v[5], c);
          o.w = pack2(v[6], v[7], c);
          *reinterpret_cast<u32x4*>(dst) = o;
        } else if constexpr (NL == 4) {
          u32x2 o;
          o.x = pack2(v[0], v[1], c);
          o.y = pack2(v[2], v[3], c);
          *reinterpret_cast<u32x2*>(dst) = o;
        } else {
          *reinterpret_cast<unsigned*>(dst) = pack2(v[0], v[1], c);
        }
      }
    }
  }
};

// One K-step's worth of operand fragments for a wave: TM A atoms, TN B atoms.
template <class Cfg>
struct Frags {
  u32x4 a[Cfg::TM], b[Cfg::TN];
};

template <class Cfg>
__device__ inline void read_frags(Frags<Cfg>& f, const char* As, const char* Bs, int a_row0,
                                  int b_row0, int chunk) {
  using At = typename Cfg::At;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
    f.a[i] = *reinterpret_cast<const u32x4*>(As + lds_off(a_row0 + i * At::M, chunk));
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j)
    f.b[j] = *reinterpret_cast<const u32x4*>(Bs + lds_off(b_row0 + j * At::N, chunk));
}

template <class Cfg, class Tag>
__device__ inline void mma_step(typename Cfg::At::acc_t (&acc)[Cfg::TM][Cfg::TN],
                                const Frags<Cfg>& f) {
  using At = typename Cfg::At;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = At::mma(Tag{}, f.a[i], f.b[j], acc[i][j]);
}

// The last K step of a masked tile on 16x16x32 atoms: only the sub-steps
// that hold valid K-values (krem of them, 1..BK) run, and a sub-step whose
// valid part is at most 16 K-values runs as v_mfma_f32_16x16x16 on its first
// half instead of multiplying 16 staged zeros. `cur` holds sub-step 0.
template <class Cfg, class Tag>
__device__ inline void k_tail(typename Cfg::At::acc_t (&acc)[Cfg::TM][Cfg::TN], Frags<Cfg>& cur,
                              const char* As, const char* Bs, int a_row0, int b_row0, int lane,
                              int krem) {
  using At = typename Cfg::At;
  constexpr int CPS = At::K / 8;
  const int koct = At::frag_koct(lane);
#pragma unroll
  for (int ks = 0; ks < Cfg::KSTEPS; ++ks) {
    const int lo = ks * At::K;
    if (lo >= krem) break;
    if (ks > 0) read_frags<Cfg>(cur, As, Bs, a_row0, b_row0, ks * CPS + koct);
    if constexpr (At::K == 32) {
      if (krem - lo <= 16) {
        // lane l: 4 K-values at lo + 4*(l >> 4), i.e. 8 bytes into chunk
        // lo/8 + (l >> 5) at byte 8*((l >> 4) & 1)
        const int chunk = lo / 8 + (lane >> 5), byte = 8 * ((lane >> 4) & 1);
        u32x2 a2[Cfg::TM], b2[Cfg::TN];
#pragma unroll
        for (int i = 0; i < Cfg::TM; ++i)
          a2[i] = *reinterpret_cast<const u32x2*>(As + lds_off(a_row0 + i * At::M, chunk) + byte);
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j)
          b2[j] = *reinterpret_cast<const u32x2*>(Bs + lds_off(b_row0 + j * At::N, chunk) + byte);
#pragma unroll
        for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
          for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = At::mma16(Tag{}, a2[i], b2[j], acc[i][j]);
        continue;
      }
    }
    mma_step<Cfg, Tag>(acc, cur);
  }
}

// -------------------------------------------------------------- epilogue ----
// Transpose a 4x4 block held by a quad of lanes (lane k of the quad holds
// x[0..3]) so that lane k ends up with element k of every lane's x: two
// exchange rounds over quad_perm DPP moves (lane ^ 2, then lane ^ 1).
__device__ inline void quad_transpose(float (&x)[4], int lane) {
  const int k = lane & 3;
  float t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float o = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x[i ^ 2]), 0x4E, 0xF, 0xF, false));
    t[i] = (((k >> 1) ^ (i >> 1)) & 1) ? o : x[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float o = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t[i ^ 1]), 0xB1, 0xF, 0xF, false));
    x[i] = ((k ^ i) & 1) ? o : t[i];
  }
}

template <int EPI>
__device__ inline float epi_one(float x, float c, float alpha, float beta) {
  if constexpr (EPI == EPI_BETA0) return alpha * x;
  else if constexpr (EPI == EPI_ACC_PLUS_C) return x + c;
  else return __builtin_fmaf(beta, c, alpha * x);
}

// D = alpha*acc + beta*C for one wave's sub-tile whose top-left output element
// is (r0, c0); C is read only for the epilogue kinds that need it.
//
// Each accumulator register group holds 4 consecutive rows of one column per
// lane. With 16-byte aligned D (and C), a quad transpose turns that into 4
// consecutive columns of one row per lane, so C is read and D is written with
// 16-byte accesses (on edge tiles too when N is a multiple of 4, each lane
// checking its row and quad); otherwise elements are written one by one with
// bounds checks.
//
// C may be D itself (the in-place form; any other overlap is rejected on the
// host), so the compiler may not move a C load above an earlier D store. The
// C values of a whole row of atoms (wide form) or of one atom (element form)
// are therefore loaded before any of their D stores: one memory round trip
// per batch instead of one per store. Each element is still read before it is
// written, by the lane that writes it.
// The C values of the wide form, in the layout store_tile uses, for callers
// that read them early (the K-split kernel, before its main loop).
template <class Cfg>
struct WideC {
  f32x4 v[Cfg::TM][Cfg::TN][Cfg::At::NACC / 4];
};
template <class Cfg>
__device__ inline void load_wide_c(WideC<Cfg>& w, const GemmArgs& p, int r0, int c0, int lane) {
  using At = typename Cfg::At;
  const int col_l = At::acc_col(lane);
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int g = 0; g < At::NACC / 4; ++g) {
        const int c = c0 + j * At::N + (col_l & ~3);
        const int r = r0 + i * At::M + At::acc_row(lane, 4 * g) + (lane & 3);
        w.v[i][j][g] = *reinterpret_cast<const f32x4*>(p.C + (int64_t)r * p.ldc + c);
      }
}

// The 16-byte form of store_tile: each lane stores 4 consecutive columns of
// a row after a quad transpose. PLAIN_STORE: plain stores (D is C, whose
// lines the C read just brought into L2); otherwise D is written once and not
// read back here, so it is streamed past the caches.
template <class Cfg, int EPI, bool MASK, bool PLAIN_STORE>
__device__ inline void store_tile_wide(typename Cfg::At::acc_t (&acc)[Cfg::TM][Cfg::TN],
                                       const GemmArgs& p, int r0, int c0, int lane,
                                       const WideC<Cfg>& pre, bool use_pre) {
  using At = typename Cfg::At;
  constexpr int NG = At::NACC / 4;  // groups of 4 rows per atom and lane
  const float alpha = p.alpha, beta = p.beta;
  const int col_l = At::acc_col(lane);
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
    f32x4 cv[Cfg::TN][NG];
    if (EPI != EPI_BETA0 && use_pre) {
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int g = 0; g < NG; ++g) cv[j][g] = pre.v[i][j][g];
    } else if constexpr (EPI != EPI_BETA0) {
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int c = c0 + j * At::N + (col_l & ~3);
          const int r = r0 + i * At::M + At::acc_row(lane, 4 * g) + (lane & 3);
          cv[j][g] = (!MASK || (r < p.M && c < p.N))
                         ? *reinterpret_cast<const f32x4*>(p.C + (int64_t)r * p.ldc + c)
                         : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int c = c0 + j * At::N + (col_l & ~3);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float x[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                      acc[i][j][4 * g + 3]};
        quad_transpose(x, lane);
        const int r = r0 + i * At::M + At::acc_row(lane, 4 * g) + (lane & 3);
        f32x4 o;
        if constexpr (EPI != EPI_BETA0) {
          o[0] = epi_one<EPI>(x[0], cv[j][g][0], alpha, beta);
          o[1] = epi_one<EPI>(x[1], cv[j][g][1], alpha, beta);
          o[2] = epi_one<EPI>(x[2], cv[j][g][2], alpha, beta);
          o[3] = epi_one<EPI>(x[3], cv[j][g][3], alpha, beta);
        } else {
          o[0] = epi_one<EPI>(x[0], 0.0f, alpha, beta);
          o[1] = epi_one<EPI>(x[1], 0.0f, alpha, beta);
          o[2] = epi_one<EPI>(x[2], 0.0f, alpha, beta);
          o[3] = epi_one<EPI>(x[3], 0.0f, alpha, beta);
        }
        if (!MASK || (r < p.M && c < p.N)) {
          f32x4* dst = reinterpret_cast<f32x4*>(p.D + (int64_t)r * p.ldd + c);
          if constexpr (PLAIN_STORE) *dst = o;
          else __builtin_nontemporal_store(o, dst);
        }
      }
    }
  }
}

// The 16-byte form for 16x16 atoms, two atoms (j, j+1) of a row of atoms at
// a time. After the quad transpose a lane holds 4 consecutive columns of one
// row in each atom, so a store instruction per atom would write 64 bytes of
// each row: half of a 128-byte line, which the memory side then fills and
// writes in part (measured at 8192^3: 1.4x D's bytes written and D's size
// again read). Lanes l and l^1, which hold rows r and r+1, swap one chunk:
// the even lane sends its atom-(j+1) chunk and the odd lane its atom-j chunk.
// Then the first instruction writes row r (even lane: its own atom-j chunk,
// odd lane: the received atom-(j+1) chunk) and the second writes row r+1,
// each lane at the column of atom j + (l & 1): 8 lanes cover the row's 32
// columns, 128 bytes. PLAIN_STORE as in store_tile_wide.
template <class Cfg, int EPI, bool MASK, bool PLAIN_STORE>
__device__ inline void store_tile_pairs16(typename Cfg::At::acc_t (&acc)[Cfg::TM][Cfg::TN],
                                          const GemmArgs& p, int r0, int c0, int lane) {
  using At = typename Cfg::At;
  static_assert(At::M == 16 && At::NACC == 4 && Cfg::TN % 2 == 0, "pairs of 16x16 atoms");
  constexpr int NP = Cfg::TN / 2;
  const float alpha = p.alpha, beta = p.beta;
  const int odd = lane & 1;
  const int col = 16 * odd + 4 * ((lane >> 2) & 3);           // within the atom pair
  const int rl = At::acc_row(lane, 0) + (lane & 3) - odd;     // row of the first store
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
    const int r = r0 + i * At::M + rl;
    f32x4 cv[NP][2];
    if constexpr (EPI != EPI_BETA0) {
      // Every C value of the row of atoms is loaded before any D store (C
      // may be D).
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int c = c0 + 32 * q + col;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          cv[q][h] = (!MASK || (r + h < p.M && c < p.N))
                         ? *reinterpret_cast<const f32x4*>(p.C + (int64_t)(r + h) * p.ldc + c)
                         : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      float x[4] = {acc[i][2 * q][0], acc[i][2 * q][1], acc[i][2 * q][2], acc[i][2 * q][3]};
      float y[4] = {acc[i][2 * q + 1][0], acc[i][2 * q + 1][1], acc[i][2 * q + 1][2],
                    acc[i][2 * q + 1][3]};
      quad_transpose(x, lane);
      quad_transpose(y, lane);
      float w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                             __builtin_bit_cast(int, odd ? x[k] : y[k]), 0xB1,
                                             0xF, 0xF, false));
      const int c = c0 + 32 * q + col;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float v = h == 0 ? (odd ? w[k] : x[k]) : (odd ? y[k] : w[k]);
          if constexpr (EPI != EPI_BETA0) o[k] = epi_one<EPI>(v, cv[q][h][k], alpha, beta);
          else o[k] = epi_one<EPI>(v, 0.0f, alpha, beta);
        }
        if (!MASK || (r + h < p.M && c < p.N)) {
          f32x4* dst = reinterpret_cast<f32x4*>(p.D + (int64_t)(r + h) * p.ldd + c);
          if constexpr (PLAIN_STORE) *dst = o;
          else __builtin_nontemporal_store(o, dst);
        }
      }
    }
  }
}

// store_tile_pairs16 where the atoms pair up, else store_tile_wide.
template <class Cfg, int EPI, bool MASK, bool PLAIN_STORE>
__device__ inline void store_tile_pairs_or_wide(typename Cfg::At::acc_t (&acc)[Cfg::TM][Cfg::TN],
                                                const GemmArgs& p, int r0, int c0, int lane) {
  if constexpr (Cfg::At::M == 16 && Cfg::TN % 2 == 0)
    store_tile_pairs16<Cfg, EPI, MASK, PLAIN_STORE>(acc, p, r0, c0, lane);
  else
    store_tile_wide<Cfg, EPI, MASK, PLAIN_STORE>(acc, p, r0, c0, lane, WideC<Cfg>{}, false);
}

template <class Cfg, int EPI, bool MASK>
__device__ inline void store_tile(typename Cfg::At::acc_t (&acc)[Cfg::TM][Cfg::TN],
                                  const GemmArgs& p, int r0, int c0, int lane,
                                  const WideC<Cfg>& pre = WideC<Cfg>{}, bool use_pre = false) {
  using At = typename Cfg::At;
  const float alpha = p.alpha, beta = p.beta;
  const int col_l = At::acc_col(lane);
  // The 16-byte form also serves masked tiles when N is a multiple of 4:
  // every quad of columns a lane stores then lies wholly inside or outside
  // N, so one predicate per lane and row decides it.
  if (p.wide_epi && (!MASK || p.N % 4 == 0)) {
    // The store kind is chosen once per tile, not per store: a branch at
    // each store measured 3-4% slower on the 128x128 kernels. Plain stores
    // where D is C gain 1.2-1.8% on the in-place accumulate at 4096^3;
    // with a separate C they lose up to 5%.
    // 16x16 atoms in pairs write whole 128-byte rows per instruction (C
    // prefetched into registers is only passed with 32x32 atoms).
    constexpr bool PAIRS = Cfg::At::M == 16 && Cfg::TN % 2 == 0;
    if constexpr (EPI != EPI_BETA0) {
      if (static_cast<const void*>(p.C) == p.D) {
        if (PAIRS && !use_pre) store_tile_pairs_or_wide<Cfg, EPI, MASK, true>(acc, p, r0, c0, lane);
        else store_tile_wide<Cfg, EPI, MASK, true>(acc, p, r0, c0, lane, pre, use_pre);
        return;
      }
    }
    if (PAIRS && !use_pre) store_tile_pairs_or_wide<Cfg, EPI, MASK, false>(acc, p, r0, c0, lane);
    else store_tile_wide<Cfg, EPI, MASK, false>(acc, p, r0, c0, lane, pre, use_pre);
    return;
  }
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int c = c0 + j * At::N + col_l;
      float cv[At::NACC];
      if constexpr (EPI != EPI_BETA0) {
#pragma unroll
        for (int v = 0; v < At::NACC; ++v) {
          const int r = r0 + i * At::M + At::acc_row(lane, v);
          cv[v] = (!MASK || (r < p.M && c < p.N)) ? p.C[(int64_t)r * p.ldc + c] : 0.0f;
        }
      }
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) {
        const int r = r0 + i * At::M + At::acc_row(lane, v);
        if (MASK && (r >= p.M || c >= p.N)) continue;
        p.D[(int64_t)r * p.ldd + c] =
            epi_one<EPI>(acc[i][j][v], EPI != EPI_BETA0 ? cv[v] : 0.0f, alpha, beta);
      }
    }
  }
}

// ---------------------------------------------------------------- kernel ----
// Pipeline per K step kt (LDS buffer b = kt & 1, the other buffer nb):
//   K sub-steps 0..KSTEPS-2: read the fragments of sub-step s+1 from b while
//     the MFMAs of sub-step s run;
//   then (all reads of b are in registers) write the staged box of step kt+1
//     into nb, barrier, issue the global loads of step kt+2, read the first
//     fragments of step kt+1 from nb, and only then run the MFMAs of the last
//     sub-step of kt, which hide that LDS latency.
// Global loads therefore have almost two K steps of MFMA work to land.
// With K groups (Cfg::KG > 1) every group runs this pipeline on its own K
// steps; all groups run the same number of steps (a group's steps past the
// end of K stage zeros, which the host guarantees by masking such shapes).
template <class Cfg, class Tag, bool TA, bool TB, bool MASK, int EPI>
__global__ void __launch_bounds__(Cfg::THREADS)
gemm_mfma_kernel(const GemmArgs p) {
  using At = typename Cfg::At;
  using acc_t = typename At::acc_t;
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];

  const int lane = threadIdx.x & 63;
  // Uniform within a wave: the K group, and with it each step's K offset and
  // the buffer resources built from it, stay scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave / (Cfg::WM * Cfg::WN);        // K group
  const int gwave = wave % (Cfg::WM * Cfg::WN);      // wave within its group
  const int tid = threadIdx.x % Cfg::GROUP_THREADS;  // thread within its group
  const int wm = gwave / Cfg::WN;
  const int wn = gwave % Cfg::WN;
  char* const smem = lds + grp * Cfg::GROUP_LDS_BYTES;

  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * Cfg::BM;
  const int n0 = tn * Cfg::BN;

  // A box rows are M indices; B box rows are N indices. A is K-contiguous
  // unless transposed; B is K-contiguous only when transposed.
  Stager<Cfg::BM, Cfg::GROUP_THREADS, !TA, MASK> sa;
  Stager<Cfg::BN, Cfg::GROUP_THREADS, TB, MASK> sb;

  acc_t acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) acc[i][j][v] = 0.0f;

  // This group's K steps: kstep(kt) is the first K index of its kt-th step.
  const int KT = ((p.K + Cfg::BK - 1) / Cfg::BK + Cfg::KG - 1) / Cfg::KG;
  auto kstep = [&](int kt) { return (kt * Cfg::KG + grp) * Cfg::BK; };
  const int a_row0 = wm * Cfg::WTM + At::frag_row(lane);
  const int b_row0 = wn * Cfg::WTN + At::frag_row(lane);
  const int koct = At::frag_koct(lane);
  constexpr int CPS = At::K / 8;  // 16-byte chunks per K sub-step

  // Masked kernel: tiles wholly inside M (N) read the whole K steps of A (B)
  // with the unmasked loads when the operand allows them.
  const bool inner_m = Cfg::INNER_PATHS && m0 + Cfg::BM <= p.M;
  const bool inner_n = Cfg::INNER_PATHS && n0 + Cfg::BN <= p.N;
  const bool a_whole = MASK && p.a_fast && inner_m, b_whole = MASK && p.b_fast && inner_n;
  // A box's pieces (8 K-values of one row for a K-contiguous operand, else 8
  // row-values of one K row) are wholly inside or outside the operand when
  // the edge that crosses them falls on a multiple of 8.
  const bool a_pieces = MASK && p.a_fast && p.a_vw == 8 &&
                        (TA ? (inner_m || p.M % 8 == 0) : p.K % 8 == 0);
  const bool b_pieces = MASK && p.b_fast && p.b_vw == 8 &&
                        (TB ? p.K % 8 == 0 : (inner_n || p.N % 8 == 0));
  // K-split tiles: group 0 reads the C it will need before the main loop,
  // so that latency overlaps the K steps instead of following the group sum.
  constexpr bool PRE_C = Cfg::KG > 1 && EPI != EPI_BETA0;
  WideC<Cfg> cpre;
  const bool pre_c = PRE_C && grp == 0 && p.wide_epi && (!MASK || (inner_m && inner_n));
  if constexpr (PRE_C) {
    if (pre_c) load_wide_c<Cfg>(cpre, p, m0 + wm * Cfg::WTM, n0 + wn * Cfg::WTN, lane);
  }
  auto load_step = [&](int k0) {
    const bool kin = k0 + Cfg::BK <= p.K;
    sa.load(p.A, p.lda, m0, p.M, k0, p.K, tid, p.a_vw, p.src32, a_whole && kin, a_pieces);
    sb.load(p.B, p.ldb, n0, p.N, k0, p.K, tid, p.b_vw, p.src32, b_whole && kin, b_pieces);
  };

  // Prologue: step 0 into buffer 0, step 1 into registers, first fragments.
  load_step(kstep(0));
  sa.store(smem, tid);
  sb.store(smem + Cfg::A_BYTES, tid);
  __syncthreads();
  if (KT > 1) load_step(kstep(1));
  Frags<Cfg> cur, nxt;
  read_frags<Cfg>(cur, smem, smem + Cfg::A_BYTES, a_row0, b_row0, koct);

  for (int kt = 0; kt < KT; ++kt) {
    const char* As = smem + (kt & 1) * Cfg::STAGE_BYTES;
    const char* Bs = As + Cfg::A_BYTES;
    // K tails on the 16x16x32 atom only: on the 32x32 atoms the tail saves
    // little and the extra control flow around 256 accumulators makes the
    // compiler spill them. A group's last step may lie wholly past K
    // (krem <= 0: nothing runs) or be whole (krem >= BK: every sub-step runs).
    if constexpr (MASK && At::K == 32) {
      if (kt == KT - 1) {
        k_tail<Cfg, Tag>(acc, cur, As, Bs, a_row0, b_row0, lane, p.K - kstep(kt));
        break;
      }
    }
#pragma unroll
    for (int ks = 0; ks < Cfg::KSTEPS - 1; ++ks) {
      read_frags<Cfg>(nxt, As, Bs, a_row0, b_row0, (ks + 1) * CPS + koct);
      mma_step<Cfg, Tag>(acc, cur);
      cur = nxt;
    }
    if (kt + 1 < KT) {
      char* nA = smem + ((kt + 1) & 1) * Cfg::STAGE_BYTES;
      sa.store(nA, tid);
      sb.store(nA + Cfg::A_BYTES, tid);
      __syncthreads();
      if (kt + 2 < KT) load_step(kstep(kt + 2));
      read_frags<Cfg>(nxt, nA, nA + Cfg::A_BYTES, a_row0, b_row0, koct);
    }
    mma_step<Cfg, Tag>(acc, cur);
    cur = nxt;
  }

  if constexpr (Cfg::KG > 1) {
    // Groups 1..KG-1 hand their accumulators to group 0 through LDS (lane-
    // major, so each store and load is one contiguous 256-byte row per
    // register); group 0 adds them in group order and runs the epilogue.
    constexpr int NREG = Cfg::TM * Cfg::TN * At::NACC;
    float* xfer = reinterpret_cast<float*>(lds);
    __syncthreads();  // every group is done reading its operand stages
    if (grp > 0) {
      float* dst = xfer + ((grp - 1) * (Cfg::WM * Cfg::WN) + gwave) * NREG * 64 + lane;
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
          for (int v = 0; v < At::NACC; ++v)
            dst[((i * Cfg::TN + j) * At::NACC + v) * 64] = acc[i][j][v];
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < Cfg::KG; ++g) {
      const float* src = xfer + ((g - 1) * (Cfg::WM * Cfg::WN) + gwave) * NREG * 64 + lane;
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
          for (int v = 0; v < At::NACC; ++v)
            acc[i][j][v] += src[((i * Cfg::TN + j) * At::NACC + v) * 64];
    }
  }

  // Tiles wholly inside M x N need no masked stores, even in the masked kernel.
  if (!MASK || (inner_m && inner_n))
    store_tile<Cfg, EPI, false>(acc, p, m0 + wm * Cfg::WTM, n0 + wn * Cfg::WTN, lane, cpre,
                                pre_c);
  else
    store_tile<Cfg, EPI, true>(acc, p, m0 + wm * Cfg::WTM, n0 + wn * Cfg::WTN, lane);
}

template <class Cfg, class Tag, bool TA, bool TB, bool MASK>
hipError_t launch_epi(const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(Cfg::THREADS);
  switch (a.epi) {
    case EPI_BETA0:
      return launch_kernel(gemm_mfma_kernel<Cfg, Tag, TA, TB, MASK, EPI_BETA0>, grid, block, s, a);
    case EPI_ACC_PLUS_C:
      return launch_kernel(gemm_mfma_kernel<Cfg, Tag, TA, TB, MASK, EPI_ACC_PLUS_C>, grid, block,
                           s, a);
    default:
      return launch_kernel(gemm_mfma_kernel<Cfg, Tag, TA, TB, MASK, EPI_GENERAL>, grid, block, s,
                           a);
  }
}

// Forms compiled: FORMS_BOTH, FORMS_MASKED (the configuration's unmasked
// calls run elsewhere) or FORMS_WHOLE (whole tiles only: the masked form
// would not fit the registers the configuration leaves); a launch request
// for a form not compiled fails.
enum CfgForms : int { FORMS_BOTH = 0, FORMS_MASKED = 1, FORMS_WHOLE = 2 };
template <class Cfg, int FORMS = FORMS_BOTH>
hipError_t launch_mfma_cfg(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                           hipStream_t s) {
  if ((FORMS == FORMS_MASKED && !masked) || (FORMS == FORMS_WHOLE && masked))
    return hipErrorInvalidValue;
#define DGT_LAUNCH_MASK(TAG, TA_, TB_)                                                \
  if constexpr (FORMS == FORMS_MASKED) return launch_epi<Cfg, TAG, TA_, TB_, true>(a, s);  \
  else if constexpr (FORMS == FORMS_WHOLE) return launch_epi<Cfg, TAG, TA_, TB_, false>(a, s); \
  else return masked ? launch_epi<Cfg, TAG, TA_, TB_, true>(a, s)                     \
                     : launch_epi<Cfg, TAG, TA_, TB_, false>(a, s)
#define DGT_LAUNCH_T(TAG)                                   \
  do {                                                      \
    if (!ta && !tb) { DGT_LAUNCH_MASK(TAG, false, false); } \
    if (!ta && tb) { DGT_LAUNCH_MASK(TAG, false, true); }   \
    if (ta && !tb) { DGT_LAUNCH_MASK(TAG, true, false); }   \
    DGT_LAUNCH_MASK(TAG, true, true);                       \
  } while (0)
  if (dtype == 0) DGT_LAUNCH_T(TagF16);
  DGT_LAUNCH_T(TagBF16);
#undef DGT_LAUNCH_T
#undef DGT_LAUNCH_MASK
}

using Cfg256 = TileCfg<256, 256, 2, 2, 32>;
using Cfg128 = TileCfg<128, 128, 2, 2, 32>;
using Cfg64 = TileCfg<64, 64, 2, 2, 16>;
using Cfg16 = TileCfg<16, 16, 1, 1, 16>;
// Under-filled grids: 32x32 tiles, K split over four (or, for long K, eight)
// one-wave groups.
using Cfg32k4 = TileCfg<32, 32, 1, 1, 32, 4>;
using Cfg32k8 = TileCfg<32, 32, 1, 1, 32, 8>;
// Skinny grids with a long K: 64x64 tiles (2x2 waves), K split over four
// groups of four waves.
using Cfg64k4 = TileCfg<64, 64, 2, 2, 16, 4>;

hipError_t launch_mfma_256(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_128(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_64(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_16(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_32k4(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_32k8(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_64k4(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);

}  // namespace dgt
