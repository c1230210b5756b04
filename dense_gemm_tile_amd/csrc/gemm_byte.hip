// Matrix-core GEMM for 1-byte operands, D = alpha*op(A)@op(B) + beta*C:
//
//  * int8 x int8 -> int32 (v_mfma_i32_32x32x32_i8): int32 C/D, integer
//    alpha/beta, all sums and the epilogue wrapping like int32 arithmetic. The
//    integer form of the same contraction (Phobos `@tensorcore`: an i8 dot
//    takes the integer tensor cores whenever its shape allows, "When it
//    declines").
//  * 8-bit floats (OCP E4M3 or E5M2) -> f32 (v_mfma_f32_32x32x64_f8f6f4, the
//    form without block scales): f32 C/D and alpha/beta, the epilogue of the 16-bit
//    kernels. The fp8 precision of the `gemm_async` variants (TVM `gemm`,
//    restated: the precision list).
//
// Both follow the contraction of TVM TIRx `gemm` ("Algorithm" steps 1-3):
//
//  * 128x128 output tile per workgroup, 4 waves (2x2) of 64x64 outputs, each a
//    2x2 block of 32x32 atoms (16 accumulators per lane per atom);
//  * K steps of 128 one-byte values: one LDS row per M (or N) index holds 128
//    bytes, eight 16-byte chunks, chunk c of row r at c ^ ((r ^ (r>>3)) & 7)
//    (the 16-bit kernels' layout, in bytes). An int8 atom (K = 32) takes 16
//    consecutive K-values per lane (lanes 0-31 the first 16, lanes 32-63 the
//    second), one ds_read_b128; an 8-bit float atom (K = 64) takes 32 (two
//    reads). Any K order shared by A and B gives the same sum, so only the
//    lane's row/column and its half of the atom's K range have to match the
//    hardware;
//  * global -> VGPR -> LDS staging, two LDS stages, the next K step loaded
//    while the current one is multiplied. K-contiguous operands move in
//    16-byte pieces when the piece is whole and aligned, bytewise otherwise;
//    M/N-contiguous operands are read 16 values along M (or N) and written
//    into their K-contiguous LDS rows byte by byte;
//  * out-of-range elements are staged as zeros (their products are zero), C
//    loads and D stores are predicated.
#include "gemm_ring.h"

#include <cstdint>
#include <type_traits>

namespace dgt {

namespace {

// Byte offset of 16-byte chunk `chunk` of LDS row `row` (128-byte rows).
__device__ inline int lds_off_b(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// int8 -> int32 atom: 32 K-values per MFMA, 16 bytes per lane.
struct KindI8 {
  static constexpr int ATOM = 32;
  using acc_t = i32x16;
  using frag_t = i32x4;
  static constexpr int KATOM = 32;
  __device__ static inline frag_t read(const char* base, int row, int ks, int half) {
    return *reinterpret_cast<const i32x4*>(base + lds_off_b(row, 2 * ks + half));
  }
  // Same read from a precomputed offset: off = lds_off_b(row, CHUNK0 * half);
  // the chunk of sub-step ks differs by bits the swizzle leaves alone.
  static constexpr int CHUNK0 = 1;
  __device__ static inline frag_t read_off(const char* base, int off, int ks) {
    return *reinterpret_cast<const i32x4*>(base + (off ^ (ks << 5)));
  }
  __device__ static inline acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
  // cbits: C[r][c] as read by epilogue() (when p.read_c).
  __device__ static inline void store(const GemmByteArgs& p, int64_t r, int c, acc_t v, int e,
                                      unsigned cbits) {
    unsigned d = (unsigned)p.alpha_i * (unsigned)v[e];
    if (p.read_c) d += (unsigned)p.beta_i * cbits;
    static_cast<int32_t*>(p.D)[r * p.ldd + c] = (int32_t)d;
  }
};

// 8-bit float atom (FMT 0: E4M3, 1: E5M2): 64 K-values per MFMA, 32 bytes per
// lane; block scales of 1 (E8M0 code 127).
template <int FMT>
struct KindF8 {
  static constexpr int ATOM = 32;
  using acc_t = f32x16_t;
  using frag_t = i32x8;
  static constexpr int KATOM = 64;
  __device__ static inline frag_t read(const char* base, int row, int ks, int half) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(base + lds_off_b(row, 4 * ks + 2 * half));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(base + lds_off_b(row, 4 * ks + 2 * half + 1));
    return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
  static constexpr int CHUNK0 = 2;
  __device__ static inline frag_t read_off(const char* base, int off, int ks) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(base + (off ^ ((4 * ks) << 4)));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(base + (off ^ ((4 * ks + 1) << 4)));
    return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
  __device__ static inline acc_t mma(frag_t a, frag_t b, acc_t c) {
    // scale operands 0: the unscaled form, as in KindF8x16
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, 0, 0, 0);
  }
  // cbits: C[r][c] as read by epilogue() (when p.read_c).
  __device__ static inline void store(const GemmByteArgs& p, int64_t r, int c, acc_t v, int e,
                                      unsigned cbits) {
    float d = p.alpha_f * v[e];
    if (p.read_c) d = __builtin_fmaf(p.beta_f, __builtin_bit_cast(float, cbits), d);
    static_cast<float*>(p.D)[r * p.ldd + c] = d;
  }
};
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

typedef int v2i __attribute__((ext_vector_type(2)));
// ds_read_b64_tr_b8 (lane layout measured with an in-bounds probe): within
// each group of 16 lanes, lane t receives byte t % 8 of the 8-byte blocks
// named by lanes 2b + t / 8, b = 0 .. 7. Lane 2b + h naming K-row k0 + b,
// columns c0 + 8h .. +7 gives lane t the 8 consecutive K-values k0 .. k0+7
// of column c0 + t.
__device__ inline v2i ds_read_tr8(const char* p) {
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p));
}

// The two-group kernel's 16x16 atoms (see gemm_mfma_pingpong.h: under the
// chip's power limit the 16-wide form clocks higher). A lane's fragment is
// 16 bytes of row (or column) l % 16; D bits are combined from accumulator
// and C bits as the 32-wide kinds' store() does.
// int8 -> int32, 16x16x64: K bytes 16 (l / 16) .. +15 of the atom's 64, so a
// 128-byte LDS row holds two sub-steps (chunk 4 ks + l / 16).
struct KindI8x16 {
  static constexpr int ATOM = 16;
  static constexpr int KIND_ID = 1;  // distinct per two-group kind (template tags)
  using acc_t = i32x4;
  using frag_t = i32x4;
  static constexpr int KATOM = 64;
  __device__ static inline frag_t read_off(const char* base, int off, int ks) {
    return *reinterpret_cast<const i32x4*>(base + (off ^ (ks << 6)));
  }
  __device__ static inline acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
  // M/N-contiguous slot (K-rows of 256 bytes): two transposed reads, K-rows
  // k .. k+7 and k+8 .. k+15 of the lane's column; sub-step ks is 64 rows on.
  __device__ static inline frag_t read_mn(const char* q, int ks) {
    const char* r = q + ks * 64 * 256;
    const v2i lo = ds_read_tr8(r), hi = ds_read_tr8(r + 8 * 256);
    return frag_t{lo.x, lo.y, hi.x, hi.y};
  }
  __device__ static inline unsigned combine(const GemmByteArgs& p, unsigned acc, unsigned c) {
    unsigned d = (unsigned)p.alpha_i * acc;
    if (p.read_c) d += (unsigned)p.beta_i * c;
    return d;
  }
};
// 8-bit float -> f32, 16x16x128 (unit block scales): 32 K bytes per lane,
// taken as chunks g and g + 4 of the 128-byte row (g = l / 16) instead of 2g
// and 2g + 1: a K order that A and B share, so the same products are summed,
// and the chunk pattern of one read is the 16-bit 16x16x32 kernel's, whose
// swizzle serves it without bank conflicts.
template <int FMT>
struct KindF8x16 {
  static constexpr int ATOM = 16;
  static constexpr int KIND_ID = 2 + FMT;
  using acc_t = f32x4;
  using frag_t = i32x8;
  static constexpr int KATOM = 128;
  __device__ static inline frag_t read_off(const char* base, int off, int) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(base + off);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(base + (off ^ 64));  // chunk g ^ 4
    return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
  // Scale operands of 0 select the form of the instruction without block
  // scales (v_mfma_f32_16x16x128_f8f6f4), which multiplies the codes as they
  // are, as unit scales would. Measured: the scaled form with unit scales
  // (127) ran 29 % slower at 8192^3 in the two-group kernel, as fast as the
  // unscaled one only when no loads were in flight; the same fragments fed
  // to two int8 MFMAs of the same total cycles ran at the unscaled speed.
  __device__ static inline acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, FMT, 0, 0, 0, 0);
  }
  // M/N-contiguous slot: K-rows 16g .. +15 and 16g + 64 .. +15 of the lane's
  // column (the same K order as read_off), four transposed reads.
  __device__ static inline frag_t read_mn(const char* q, int) {
    const v2i a = ds_read_tr8(q), b = ds_read_tr8(q + 8 * 256);
    const v2i c = ds_read_tr8(q + 64 * 256), d = ds_read_tr8(q + 72 * 256);
    return frag_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
  }
  __device__ static inline unsigned combine(const GemmByteArgs& p, unsigned acc, unsigned c) {
    float d = p.alpha_f * __builtin_bit_cast(float, acc);
    if (p.read_c) d = __builtin_fmaf(p.beta_f, __builtin_bit_cast(float, c), d);
    return __builtin_bit_cast(unsigned, d);
  }
};

// Epilogue of a wave's sub-tile of 16x16 atoms on whole tiles with 16-byte
// C/D rows, two atoms at a time, as store_tile_pairs16 does for the float
// kernels: after a quad transpose each lane holds 4 consecutive columns of one
// row per atom; lanes l and l^1 swap one chunk so that every store
// instruction writes whole 128-byte rows. All C values of a row of atoms are
// read before its first D store (C may be D).
// MASK (edge tiles, N a multiple of 4): C is read and D written only at rows
// below M and column quads below N.
template <class Kind, class C, bool MASK = false>
__device__ inline void byte_store_pairs16(const GemmByteArgs& p, int r0, int c0,
                                          typename Kind::acc_t (&acc)[C::TM][C::TN], int lane) {
  static_assert(Kind::ATOM == 16 && C::TN % 2 == 0, "pairs of 16x16 atoms");
  constexpr int NP = C::TN / 2;
  const int odd = lane & 1;
  const int col = 16 * odd + 4 * ((lane >> 2) & 3);
  const int rl = 4 * (lane >> 4) + (lane & 3) - odd;
  const bool c_is_d = p.read_c && p.C == static_cast<const void*>(p.D);
  const unsigned* Cb = static_cast<const unsigned*>(p.C);
  unsigned* Db = static_cast<unsigned*>(p.D);
  // (MASK) C and D element by element: rows not 16-byte aligned, or N % 4 != 0
  const bool scalar = MASK && p.cd_scalar;  // uniform
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int r = r0 + 16 * i + rl;
    u32x4_t cv[NP][2];
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cc = c0 + 32 * q + col;
        if (scalar) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            cv[q][h][k] = p.read_c && r + h < p.M && cc + k < p.N
                              ? Cb[(int64_t)(r + h) * p.ldc + cc + k]
                              : 0u;
        } else {
          cv[q][h] = p.read_c && (!MASK || (r + h < p.M && cc < p.N))
                         ? *reinterpret_cast<const u32x4_t*>(Cb + (int64_t)(r + h) * p.ldc + cc)
                         : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      // (whole-vector casts: a bit cast of one element of a vector reference
      // compiled to reads of element 0)
      const f32x4 xv = __builtin_bit_cast(f32x4, acc[i][2 * q]);
      const f32x4 yv = __builtin_bit_cast(f32x4, acc[i][2 * q + 1]);
      float x[4] = {xv[0], xv[1], xv[2], xv[3]};
      float y[4] = {yv[0], yv[1], yv[2], yv[3]};
      quad_transpose(x, lane);
      quad_transpose(y, lane);
      float w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                             __builtin_bit_cast(int, odd ? x[k] : y[k]), 0xB1,
                                             0xF, 0xF, false));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4_t o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float v = h == 0 ? (odd ? w[k] : x[k]) : (odd ? y[k] : w[k]);
          o[k] = Kind::combine(p, __builtin_bit_cast(unsigned, v), cv[q][h][k]);
        }
        if (scalar) {
          const int cc = c0 + 32 * q + col;
          if (r + h < p.M) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (cc + k < p.N) Db[(int64_t)(r + h) * p.ldd + cc + k] = o[k];
          }
          continue;
        }
        if (MASK && !(r + h < p.M && c0 + 32 * q + col < p.N)) continue;
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(Db + (int64_t)(r + h) * p.ldd + c0 + 32 * q + col);
        if (c_is_d) *dst = o;
        else __builtin_nontemporal_store(o, dst);
      }
    }
  }
}

// Epilogue of one 32x32 atom whose top-left output element is (r0, c0): lane
// l's accumulator v is row 8*(v/4) + 4*(l/32) + v%4, column l%32. C (32-bit
// int or float, read as raw bits) may be D itself, so the compiler may not
// move a C load above an earlier D store: all of the atom's C values are read
// before its first store, one memory round trip per atom instead of per
// element. Each element is read before it is written, by the lane that
// writes it.
template <class Kind, bool MASK>
__device__ inline void epilogue(const GemmByteArgs& p, int r0, int c0,
                                const typename Kind::acc_t& acc, int lane) {
  unsigned cb[16];
  const int c = c0 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = r0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    const bool in = !MASK || (r < p.M && c < p.N);
    cb[v] = (p.read_c && in) ? static_cast<const unsigned*>(p.C)[(int64_t)r * p.ldc + c] : 0u;
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = r0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (!MASK || (r < p.M && c < p.N)) Kind::store(p, r, c, acc, v, cb[v]);
  }
}

constexpr int kBM = 128, kBN = 128, kBK = 128, kThreads = 256;
constexpr int kTM = 2, kTN = 2;           // atoms per wave
constexpr int kBox = kBM * kBK;           // bytes of one operand box (BM == BN)
constexpr int kStage = 2 * kBox;
constexpr int kPieces = kBox / 16 / kThreads;  // 16-byte pieces per thread per operand: 4

// One operand's 128 x 128 box (rows: M or N indices; K) at (r0, k0).
// KCONTIG: element (r, k) is X[r * ld + k]; otherwise X[k * ld + r].
template <bool KCONTIG>
struct ByteStager {
  u32x4_t v[kPieces];

  __device__ static inline u32x4_t load_bytes(const int8_t* p, int n, int64_t stride) {
    unsigned w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const unsigned b = q < n ? (unsigned)(uint8_t)p[q * stride] : 0u;
      w[q >> 2] |= b << (8 * (q & 3));
    }
    return u32x4_t{w[0], w[1], w[2], w[3]};
  }

  // vec16: the operand's base and row pitch are multiples of 16 bytes.
  __device__ inline void load(const int8_t* __restrict__ X, int64_t ld, int r0, int rlim, int k0,
                              int klim, int tid, bool vec16) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int id = tid + i * kThreads;
      if constexpr (KCONTIG) {
        // piece id: row id / 8, K chunk id % 8
        const int r = r0 + (id >> 3), k = k0 + ((id & 7) << 4);
        const int8_t* p = X + (int64_t)r * ld + k;
        if (r < rlim && k < klim) {
          v[i] = (vec16 && k + 16 <= klim) ? *reinterpret_cast<const u32x4_t*>(p)
                                            : load_bytes(p, klim - k, 1);
        } else {
          v[i] = u32x4_t{0u, 0u, 0u, 0u};
        }
      } else {
        // piece id: K row id / 8, 16 rows of M (or N) starting at 16 * (id % 8)
        const int k = k0 + (id >> 3), r = r0 + ((id & 7) << 4);
        const int8_t* p = X + (int64_t)k * ld + r;
        if (k < klim && r < rlim) {
          v[i] = (vec16 && r + 16 <= rlim) ? *reinterpret_cast<const u32x4_t*>(p)
                                            : load_bytes(p, rlim - r, 1);
        } else {
          v[i] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  }

  __device__ inline void store(char* __restrict__ lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int id = tid + i * kThreads;
      if constexpr (KCONTIG) {
        *reinterpret_cast<u32x4_t*>(lds + lds_off_b(id >> 3, id & 7)) = v[i];
      } else {
        // byte q of the piece is element (row 16 * (id % 8) + q, K id / 8)
        const int kk = id >> 3, rb = (id & 7) << 4;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const uint8_t b = (uint8_t)(v[i][q >> 2] >> (8 * (q & 3)));
          lds[lds_off_b(rb + q, kk >> 4) + (kk & 15)] = (char)b;
        }
      }
    }
  }
};

template <class Kind, bool TA, bool TB>
__global__ void __launch_bounds__(kThreads) gemm_byte_kernel(const GemmByteArgs p) {
  using acc_t = typename Kind::acc_t;
  using frag_t = typename Kind::frag_t;
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  ByteStager<!TA> sa;  // A is K-contiguous unless transposed
  ByteStager<TB> sb;   // B is K-contiguous only when transposed
  const int8_t* A = static_cast<const int8_t*>(p.A);
  const int8_t* B = static_cast<const int8_t*>(p.B);
  acc_t acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  const int KT = (p.K + kBK - 1) / kBK;
  const int a_row0 = wm * 64 + (lane & 31), b_row0 = wn * 64 + (lane & 31);
  const int half = lane >> 5;  // which half of an atom's K range this lane holds

  if (KT > 0) {
    sa.load(A, p.lda, m0, p.M, 0, p.K, tid, p.a_vec16);
    sb.load(B, p.ldb, n0, p.N, 0, p.K, tid, p.b_vec16);
    sa.store(smem, tid);
    sb.store(smem + kBox, tid);
    __syncthreads();
  }
  for (int kt = 0; kt < KT; ++kt) {
    const char* As = smem + (kt & 1) * kStage;
    const char* Bs = As + kBox;
    if (kt + 1 < KT) {
      sa.load(A, p.lda, m0, p.M, (kt + 1) * kBK, p.K, tid, p.a_vec16);
      sb.load(B, p.ldb, n0, p.N, (kt + 1) * kBK, p.K, tid, p.b_vec16);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / Kind::KATOM; ++ks) {
      frag_t fa[kTM], fb[kTN];
#pragma unroll
      for (int i = 0; i < kTM; ++i) fa[i] = Kind::read(As, a_row0 + 32 * i, ks, half);
#pragma unroll
      for (int j = 0; j < kTN; ++j) fb[j] = Kind::read(Bs, b_row0 + 32 * j, ks, half);
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = Kind::mma(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < KT) {
      char* nA = smem + ((kt + 1) & 1) * kStage;
      sa.store(nA, tid);
      sb.store(nA + kBox, tid);
    }
    __syncthreads();
  }

  // Epilogue, atom by atom (masked at the edges).
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
      epilogue<Kind, true>(p, m0 + wm * 64 + 32 * i, n0 + wn * 64 + 32 * j, acc[i][j], lane);
}

// Whole 256x256 tiles of the NT layout on the two-group ping-pong design of
// the 16-bit kernels (gemm_mfma_pingpong.h): a K slice is 128 bytes of each
// row, the same bytes per slice and the same LDS ring, loads and phases; only
// the atom (int8 or 8-bit float), the fragment reads and the epilogue differ.
// A slice is 4 int8 or 2 fp8 sub-steps of 8 MFMAs per wave, each MFMA twice
// the 16-bit one's work at twice its rate, so a compute phase stays about
// 1024 cycles.
// An M/N-contiguous 1-byte operand of the two-group kernel (A stored [K][M]
// or B stored [K][N]): a slot is 128 K-rows of 256 bytes (the tile's 256
// M or N values); chunk c (16 bytes) of row r sits at c ^ s(r),
// s(r) = (r & 7) ^ 8 r4. A transposed read touches 8 consecutive rows of one
// chunk per 16 lanes (rows 16g .. 16g + 7 for lane group g); the swizzle puts
// those 8 rows, and the next group's, on all 64 banks. Instruction i of wave
// lw fills K-rows 32 lw + 4i .. +3, lane l chunk slot l % 16 of row
// 32 lw + 4i + l / 16.
// MASK (edge tiles): pieces whose columns start at or past the operand's
// M (or N), or whose K-row is at or past K, read as zeros (out-of-range
// offset from a resource that ends at the operand's last byte); M (or N)
// must then be a multiple of 16. TAG is unused: it gives each masked kernel
// its own specialization (this compiler's host pass dropped the kernels
// that shared one with an earlier kernel).
template <int NFRAG, bool MASK = false, int TAG = 0>
struct PpByteMN {
  const char* base;  // tile's first column (M or N index), K = 0
  int64_t ld;        // row pitch in bytes
  int voff[4];       // by i & 1 and i >= 4 (they set r & 7 and bit 4 of r)
  int off[NFRAG];    // transposed-read offset of each atom, sub-step 0
  int ccol[4];       // (MASK) first column of the piece of voff[q], from the tile's
  int crem, krem0;   // (MASK) columns left from the tile's first column; K-rows
                     //    left from this lane's first K-row of slice 0 (K - 32 lw - l/16)
  int klim;          // (MASK) K

  __device__ static inline int swz(int r) { return (r & 7) ^ (8 * ((r >> 4) & 1)); }
  __device__ inline void init_load(const void* X, int64_t ld_, int c0, int lw, int lane,
                                   int clim = 0, int K = 0) {
    base = static_cast<const char*>(X) + c0;
    ld = ld_;
    const int rsub = lane >> 4, p = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int chunk = p ^ swz(4 * (q & 1) + rsub + 16 * (q >> 1));
      voff[q] = (int)((32 * lw + rsub) * ld) + (chunk << 4);
      ccol[q] = chunk << 4;
    }
    crem = clim - c0;
    krem0 = K - 32 * lw - rsub;
    klim = K;
  }
  __device__ __forceinline__ void issue(char* slot, int lw, int i, int slice) const {
    // the slice's first K-row is folded into the resource base
    const char* b = base + (int64_t)slice * 128 * ld;
    const int q = (i & 1) | ((i >= 4) << 1);
    if constexpr (!MASK) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(b), (pp_lds_ptr_t)(slot + (lw * 8 + i) * 1024),
                                               16, voff[q], (int)(4 * i * ld), 0, 0);
    } else {
      // This lane's K-row: slice*128 + 32 lw + 4 i + l/16; the record count
      // ends at the operand's last byte (K-row K-1, column clim-1), counted
      // from b, so the offsets stay in 32 bits with nothing in soffset.
      const int krem = krem0 - slice * 128 - 4 * i;
      const int voffm = (krem > 0 && ccol[q] < crem) ? voff[q] + (int)(4 * i * ld) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc_n(b, nrec_slice(slice)),
                                               (pp_lds_ptr_t)(slot + (lw * 8 + i) * 1024), 16, voffm,
                                               0, 0, 0);
    }
  }
  // Record count from the slice's base to the end of the operand's last
  // K-row's valid columns.
  __device__ inline unsigned nrec_slice(int slice) const {
    const int64_t n = (int64_t)(klim - 1 - slice * 128) * ld + crem;
    return n <= 0 ? 0u : (n > 0x7FFFFFFC ? 0x7FFFFFFCu : (unsigned)n);
  }
  // Lane l (group g = l / 16, t = l % 16) names K-row k = 16 g + t / 2,
  // columns col0 + 8 (t & 1) .. +7 of atom t's 16 columns.
  __device__ inline void init_read(int col0, int lane) {
    const int g = lane >> 4, t = lane & 15;
    const int k = 16 * g + (t >> 1);
#pragma unroll
    for (int a = 0; a < NFRAG; ++a) {
      const int col = col0 + 16 * a;
      off[a] = k * 256 + (((col >> 4) ^ swz(k)) << 4) + 8 * (t & 1);
    }
  }
};

// Masked loads of a K-contiguous 1-byte operand on edge tiles of the
// two-group kernel: the LDS placement of PpOperand<false, N, 16> with 1-byte
// elements (instruction i of wave lw: rows 64 lw + 8i .. +7 of the tile,
// lane l chunk slot l % 8 of row 64 lw + 8i + l/8), but each piece addressed
// through the voffset alone from the tile's first row, so that pieces in
// rows at or past the operand's last, or starting at or past K, read as
// zeros (out-of-range offset). K must be a multiple of 16.
struct PpByteKMasked {
  const char* base;  // tile's first row, K = 0
  unsigned nrec;     // bytes from base to the operand's last byte
  int ld, row, c0, c1, rrem, klim;

  __device__ inline void init_load(const void* X, int64_t ld_, int r0, int rlim, int K, int lw,
                                   int lane) {
    base = static_cast<const char*>(X) + (int64_t)r0 * ld_;
    ld = (int)ld_;
    klim = K;
    rrem = rlim - r0;
    row = lw * 64 + (lane >> 3);
    c0 = (lane & 7) ^ PpOperand<false, 1, 16>::swz(lane >> 3);
    c1 = (lane & 7) ^ PpOperand<false, 1, 16>::swz(8 + (lane >> 3));
    const int64_t n = rrem > 0 ? (int64_t)(rrem - 1) * ld_ + K : 0;
    nrec = n > 0x7FFFFFFC ? 0x7FFFFFFCu : (unsigned)n;
  }
  __device__ __forceinline__ void issue(char* slot, int lw, int i, int slice) const {
    const int r = row + 8 * i;
    const int k = slice * 128 + (((i & 1) ? c1 : c0) << 4);
    const int voff = (r < rrem && k < klim) ? r * ld + k : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc_n(base, nrec),
                                             (pp_lds_ptr_t)(slot + (lw * 8 + i) * 1024), 16, voff, 0,
                                             0, 0);
  }
};

template <class Kind>
struct PpByteFrags {
  typename Kind::frag_t a[PingPongCfgT<Kind::ATOM>::TM], b[PingPongCfgT<Kind::ATOM>::TN];
};

// Fragment offset (sub-step 0) of the atom whose first row of the slot is
// row0: 32-wide kinds take K half l / 32 of a row l % 32 (chunk CHUNK0 *
// half), 16-wide ones chunk l / 16 of row l % 16, with their swizzles.
template <class Kind>
__device__ inline int pp_byte_frag_off(int row0, int lane) {
  if constexpr (Kind::ATOM == 16)
    return PpOperand<false, 1, 16>::lds_off(row0 + (lane & 15), lane >> 4);
  else
    return lds_off_b(row0 + (lane & 31), Kind::CHUNK0 * (lane >> 5));
}

// AMN / BMN: A stored [K][M] / B stored [K][N] (16-wide kinds only). MASK:
// edge tiles (M, N not multiples of 256, K of 128): pieces outside the
// operands read as zeros, C and D accessed inside M x N only (K a multiple
// of 16, N of 4, and the contiguous dimension of an M/N-contiguous operand
// of 16).
template <class Kind, bool AMN, bool BMN, bool MASK = false>
__global__ void __launch_bounds__(PingPongCfg::THREADS) gemm_pp_byte_kernel(const GemmByteArgs p) {
  static_assert(Kind::ATOM == 16 || (!AMN && !BMN), "M/N-contiguous operands use 16-wide atoms");
  static_assert(Kind::ATOM == 16 || !MASK, "edge tiles use 16-wide atoms");
  using C = PingPongCfgT<Kind::ATOM>;
  using At = typename C::At;
  using acc_t = typename Kind::acc_t;
  constexpr int KS = 128 / Kind::KATOM;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2, lw = wave & 3;
  const int wm = group, wn = lw;
  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  using OpKA = std::conditional_t<MASK, PpByteKMasked, PpOperand<false, C::TM, Kind::ATOM>>;
  using OpKB = std::conditional_t<MASK, PpByteKMasked, PpOperand<false, C::TN, Kind::ATOM>>;
  // (the tag: one specialization per masked kernel, see PpByteMN)
  constexpr int TAG = MASK ? 4 * Kind::KIND_ID + 2 * AMN + BMN : 0;
  using OpA = std::conditional_t<AMN, PpByteMN<C::TM, MASK, TAG>, OpKA>;
  using OpB = std::conditional_t<BMN, PpByteMN<C::TN, MASK, TAG>, OpKB>;
  OpA a;
  OpB b;
  int offA[C::TM], offB[C::TN];  // fragment offsets within a slot, sub-step 0
  if constexpr (AMN) {
    a.init_load(p.A, p.lda, m0, lw, lane, p.M, p.K);
    a.init_read(wm * C::WTM, lane);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) offA[i] = a.off[i];
  } else {
    if constexpr (MASK) a.init_load(p.A, p.lda, m0, p.M, p.K, lw, lane);
    else a.init_load(p.A, p.lda, m0, lw, lane, 1);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) offA[i] = pp_byte_frag_off<Kind>(wm * C::WTM + At::M * i, lane);
  }
  if constexpr (BMN) {
    b.init_load(p.B, p.ldb, n0, lw, lane, p.N, p.K);
    b.init_read(wn * C::WTN, lane);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) offB[j] = b.off[j];
  } else {
    if constexpr (MASK) b.init_load(p.B, p.ldb, n0, p.N, p.K, lw, lane);
    else b.init_load(p.B, p.ldb, n0, lw, lane, 1);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) offB[j] = pp_byte_frag_off<Kind>(wn * C::WTN + At::N * j, lane);
  }
  auto read_a = [&](const char* slot, int i, int ks) {
    if constexpr (AMN) return Kind::read_mn(slot + offA[i], ks);
    else return Kind::read_off(slot, offA[i], ks);
  };
  auto read_b = [&](const char* slot, int j, int ks) {
    if constexpr (BMN) return Kind::read_mn(slot + offB[j], ks);
    else return Kind::read_off(slot, offB[j], ks);
  };

  acc_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) acc[i][j][v] = 0;

  auto issue = [&](const OpA& x, int slice, int slot) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) x.issue(smem + slot * C::SLOT_BYTES, lw, i, slice);
  };
  auto issue_b = [&](int slice, int slot) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) b.issue(smem + slot * C::SLOT_BYTES, lw, i, slice);
  };

  // Phases as in pp_mainloop: group 0 reads slice s in phase 2s+1 and
  // multiplies it in 2s+2, group 1 one phase later; A of slice t in slot
  // 2t % 5 (loaded by group 1), B in slot (2t+1) % 5 (loaded by group 0).
  const int KT = MASK ? (p.K + 127) / 128 : p.K / 128;
  if (group == 1) {
    issue(a, 0, 0);
    if (KT > 1) {
      issue(a, 1, 2);
      pp_wait_vm<C::LOADS>();
    } else {
      pp_wait_vm<0>();
    }
  } else {
    issue_b(0, 1);
    pp_wait_vm<0>();
  }
  pp_barrier();
  if (group == 1) {
    pp_wait_vm<0>();
    pp_barrier();
  }
  PpByteFrags<Kind> f[KS];
  int h = 0;
  for (int s = 0; s < KT; ++s) {
    if constexpr (AMN) {
      asm volatile("" : "+v"(a.voff[0]), "+v"(a.voff[1]), "+v"(a.voff[2]), "+v"(a.voff[3]));
    } else {
      asm volatile("" : "+v"(a.row), "+v"(a.c0));
      if constexpr (Kind::ATOM == 16) asm volatile("" : "+v"(a.c1));
    }
    if constexpr (BMN) {
      asm volatile("" : "+v"(b.voff[0]), "+v"(b.voff[1]), "+v"(b.voff[2]), "+v"(b.voff[3]));
    } else {
      asm volatile("" : "+v"(b.row), "+v"(b.c0));
      if constexpr (Kind::ATOM == 16) asm volatile("" : "+v"(b.c1));
    }
#pragma unroll
    for (int i = 0; i < C::TM; ++i) asm volatile("" : "+v"(offA[i]));
#pragma unroll
    for (int j = 0; j < C::TN; ++j) asm volatile("" : "+v"(offB[j]));
    const int sa = h, sb = h == 4 ? 0 : h + 1;
    const char* pa = smem + sa * C::SLOT_BYTES;
    const char* pb = smem + sb * C::SLOT_BYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) f[ks].a[i] = read_a(pa, i, ks);
#pragma unroll
      for (int j = 0; j < C::TN; ++j) f[ks].b[j] = read_b(pb, j, ks);
    }
    if (group == 0) {
      if (s + 1 < KT) issue_b(s + 1, h >= 2 ? h - 2 : h + 3);
      pp_wait_lgkm0();
    } else {
      const bool ld = s + 2 < KT;
      if (ld) issue(a, s + 2, h >= 1 ? h - 1 : h + 4);
      if (ld) pp_wait_vm_lgkm0<C::LOADS>();
      else pp_wait_vm_lgkm0<0>();
    }
    pp_barrier();
    // The K sub-steps of one accumulator back to back, as in the 16-bit
    // kernel (an MFMA that takes the previous one's output as its accumulator
    // issues faster than one that reads another accumulator).
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc[i][j] = Kind::mma(f[ks].a[i], f[ks].b[j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    if (group == 0) pp_wait_vm<0>();
    pp_barrier();
    h = h >= 3 ? h - 3 : h + 2;
  }
  if (group == 0) pp_barrier();

  if constexpr (Kind::ATOM == 16) {
    byte_store_pairs16<Kind, C, MASK>(p, m0 + wm * C::WTM, n0 + wn * C::WTN, acc, lane);
  } else {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        epilogue<Kind, false>(p, m0 + wm * C::WTM + 32 * i, n0 + wn * C::WTN + 32 * j, acc[i][j],
                              lane);
  }
}

// Kind: the 128x128 kernel's 32-wide atom; KindPP: the two-group kernel's.
template <class Kind, class KindPP>
hipError_t launch_kind(bool ta, bool tb, const GemmByteArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n);
  if (a.pingpong == 2) {  // edge tiles
    const dim3 block(PingPongCfg::THREADS);
    if (!ta && tb)
      return launch_kernel(gemm_pp_byte_kernel<KindPP, false, false, true>, grid, block, s, a);
    if (!ta && !tb)
      return launch_kernel(gemm_pp_byte_kernel<KindPP, false, true, true>, grid, block, s, a);
    if (ta && tb)
      return launch_kernel(gemm_pp_byte_kernel<KindPP, true, false, true>, grid, block, s, a);
    return launch_kernel(gemm_pp_byte_kernel<KindPP, true, true, true>, grid, block, s, a);
  }
  if (a.pingpong) {
    const dim3 block(PingPongCfg::THREADS);
    // A is M-contiguous when stored transposed; B is N-contiguous when not.
    if (!ta && tb) return launch_kernel(gemm_pp_byte_kernel<KindPP, false, false>, grid, block, s, a);
    if (!ta && !tb) return launch_kernel(gemm_pp_byte_kernel<KindPP, false, true>, grid, block, s, a);
    if (ta && tb) return launch_kernel(gemm_pp_byte_kernel<KindPP, true, false>, grid, block, s, a);
    return launch_kernel(gemm_pp_byte_kernel<KindPP, true, true>, grid, block, s, a);
  }
  const dim3 block(kThreads);
  if (!ta && tb) return launch_kernel(gemm_byte_kernel<Kind, false, true>, grid, block, s, a);
  if (!ta && !tb) return launch_kernel(gemm_byte_kernel<Kind, false, false>, grid, block, s, a);
  if (ta && tb) return launch_kernel(gemm_byte_kernel<Kind, true, true>, grid, block, s, a);
  return launch_kernel(gemm_byte_kernel<Kind, true, false>, grid, block, s, a);
}

}  // namespace

hipError_t launch_byte(int kind, bool ta, bool tb, const GemmByteArgs& a, hipStream_t s) {
  if (kind == BYTE_I8) return launch_kind<KindI8, KindI8x16>(ta, tb, a, s);
  if (kind == BYTE_F8E4M3) return launch_kind<KindF8<0>, KindF8x16<0>>(ta, tb, a, s);
  return launch_kind<KindF8<1>, KindF8x16<1>>(ta, tb, a, s);
}

int byte_tile_m() { return kBM; }
int byte_tile_n() { return kBN; }
int byte_pp_tile() { return PingPongCfg::BM; }

}  // namespace dgt
