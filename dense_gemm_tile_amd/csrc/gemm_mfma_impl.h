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
//  * global -> VGPR -> LDS staging with 128-bit loads, two LDS stages over K
//    (load stage k+1 while computing stage k, one barrier per K step);
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
template <int BM_, int BN_, int WM_, int WN_, int ATOM_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int THREADS = WM * WN * 64;
  using At = Atom<ATOM_>;
  static constexpr int WTM = BM / WM, WTN = BN / WN;     // one wave's sub-tile
  static constexpr int TM = WTM / At::M, TN = WTN / At::N;  // atoms per wave
  static constexpr int KSTEPS = BK / At::K;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static_assert(WTM % At::M == 0 && WTN % At::N == 0, "wave tile must hold whole atoms");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
};

// Byte offset of 16-byte chunk `chunk` (0..7) of LDS row `row` (128 bytes).
__device__ static inline int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// --------------------------------------------------------------- staging ----
// One operand's R x 64 box (R rows of M or N, 64 K-values) per K step.
// KCONTIG: element (r, k) is X[(r0 + r) * ld + k0 + k]  (A with transA = 0,
//          B with transB = 1); otherwise X[(k0 + k) * ld + r0 + r].
// Each thread moves NL 16-byte pieces: for KCONTIG, NL chunks of 8 K-values;
// otherwise one block of NL K-rows x 8 row-values, transposed in registers.
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

  // rlim / klim: number of valid rows / K-values of the whole operand.
  __device__ inline void load(const uint16_t* __restrict__ X, int64_t ld, int r0, int rlim,
                              int k0, int klim, int tid) {
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int id = tid + i * THREADS;
        const int r = r0 + (id >> 3);
        const int k = k0 + ((id & 7) << 3);
        const uint16_t* p = X + (int64_t)r * ld + k;
        if (!MASK) {
          v[i] = *reinterpret_cast<const u32x4*>(p);
        } else if (r < rlim && k + 8 <= klim) {
          v[i] = *reinterpret_cast<const u32x4*>(p);
        } else if (r < rlim && k < klim) {
          v[i] = load_partial(p, klim - k);
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
        const uint16_t* p = X + (int64_t)k * ld + r;
        if (!MASK) {
          v[j] = *reinterpret_cast<const u32x4*>(p);
        } else if (k < klim && r + 8 <= rlim) {
          v[j] = *reinterpret_cast<const u32x4*>(p);
        } else if (k < klim && r < rlim) {
          v[j] = load_partial(p, rlim - r);
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

// ---------------------------------------------------------------- kernel ----
template <class Cfg, class Tag, bool TA, bool TB, bool MASK>
__global__ void __launch_bounds__(Cfg::THREADS)
gemm_mfma_kernel(const GemmArgs p) {
  using At = typename Cfg::At;
  using acc_t = typename At::acc_t;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / Cfg::WN;
  const int wn = wave % Cfg::WN;

  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * Cfg::BM;
  const int n0 = tn * Cfg::BN;

  // A box rows are M indices; B box rows are N indices. A is K-contiguous
  // unless transposed; B is K-contiguous only when transposed.
  Stager<Cfg::BM, Cfg::THREADS, !TA, MASK> sa;
  Stager<Cfg::BN, Cfg::THREADS, TB, MASK> sb;
  const uint16_t* Ap = static_cast<const uint16_t*>(p.A);
  const uint16_t* Bp = static_cast<const uint16_t*>(p.B);

  acc_t acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) acc[i][j][v] = 0.0f;

  const int KT = (p.K + Cfg::BK - 1) / Cfg::BK;

  sa.load(Ap, p.lda, m0, p.M, 0, p.K, tid);
  sb.load(Bp, p.ldb, n0, p.N, 0, p.K, tid);
  sa.store(smem, tid);
  sb.store(smem + Cfg::A_BYTES, tid);
  __syncthreads();

  // Fragment row offsets (bytes are computed per K step from these).
  const int a_row0 = wm * Cfg::WTM + At::frag_row(lane);
  const int b_row0 = wn * Cfg::WTN + At::frag_row(lane);
  const int koct = At::frag_koct(lane);

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      const int k0 = (kt + 1) * Cfg::BK;
      sa.load(Ap, p.lda, m0, p.M, k0, p.K, tid);
      sb.load(Bp, p.ldb, n0, p.N, k0, p.K, tid);
    }
    const char* As = smem + cur * Cfg::STAGE_BYTES;
    const char* Bs = As + Cfg::A_BYTES;
#pragma unroll
    for (int ks = 0; ks < Cfg::KSTEPS; ++ks) {
      const int chunk = ks * (At::K / 8) + koct;
      u32x4 a[Cfg::TM], b[Cfg::TN];
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(As + lds_off(a_row0 + i * At::M, chunk));
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
        b[j] = *reinterpret_cast<const u32x4*>(Bs + lds_off(b_row0 + j * At::N, chunk));
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = At::mma(Tag{}, a[i], b[j], acc[i][j]);
    }
    if (more) {
      char* nxt = smem + (cur ^ 1) * Cfg::STAGE_BYTES;
      sa.store(nxt, tid);
      sb.store(nxt + Cfg::A_BYTES, tid);
    }
    __syncthreads();
  }

  // Epilogue: D = alpha*acc + beta*C, once per output element.
  const float alpha = p.alpha, beta = p.beta;
  const int col_l = At::acc_col(lane);
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int cbase = n0 + wn * Cfg::WTN + j * At::N + col_l;
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) {
        const int r = m0 + wm * Cfg::WTM + i * At::M + At::acc_row(lane, v);
        const int c = cbase;
        if (MASK && (r >= p.M || c >= p.N)) continue;
        const float x = acc[i][j][v];
        float* dp = p.D + (int64_t)r * p.ldd + c;
        if (p.epi == EPI_BETA0) {
          *dp = alpha * x;
        } else {
          const float cv = p.C[(int64_t)r * p.ldc + c];
          *dp = (p.epi == EPI_ACC_PLUS_C) ? (x + cv) : __builtin_fmaf(beta, cv, alpha * x);
        }
      }
    }
  }
}

template <class Cfg>
hipError_t launch_mfma_cfg(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                           hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(Cfg::THREADS);
#define DGT_LAUNCH(TAG, TA_, TB_, MASK_) \
  gemm_mfma_kernel<Cfg, TAG, TA_, TB_, MASK_><<<grid, block, 0, s>>>(a)
#define DGT_LAUNCH_MASK(TAG, TA_, TB_)                 \
  do {                                                 \
    if (masked) DGT_LAUNCH(TAG, TA_, TB_, true);       \
    else DGT_LAUNCH(TAG, TA_, TB_, false);             \
  } while (0)
#define DGT_LAUNCH_T(TAG)                                  \
  do {                                                     \
    if (!ta && !tb) DGT_LAUNCH_MASK(TAG, false, false);    \
    else if (!ta && tb) DGT_LAUNCH_MASK(TAG, false, true); \
    else if (ta && !tb) DGT_LAUNCH_MASK(TAG, true, false); \
    else DGT_LAUNCH_MASK(TAG, true, true);                 \
  } while (0)
  if (dtype == 0) DGT_LAUNCH_T(TagF16);
  else DGT_LAUNCH_T(TagBF16);
#undef DGT_LAUNCH_T
#undef DGT_LAUNCH_MASK
#undef DGT_LAUNCH
  return hipGetLastError();
}

using Cfg256 = TileCfg<256, 256, 2, 2, 32>;
using Cfg128 = TileCfg<128, 128, 2, 2, 32>;
using Cfg64 = TileCfg<64, 64, 2, 2, 16>;
using Cfg16 = TileCfg<16, 16, 1, 1, 16>;

hipError_t launch_mfma_256(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_128(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_64(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);
hipError_t launch_mfma_16(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a, hipStream_t s);

}  // namespace dgt
