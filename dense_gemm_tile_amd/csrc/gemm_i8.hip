// int8 x int8 -> int32 matrix-core GEMM: D = alpha*op(A)@op(B) + beta*C with
// int32 C/D and integer alpha/beta, all sums and the epilogue wrapping like
// int32 arithmetic.
//
// The integer form of the same contraction (TVM TIRx `gemm`: "Algorithm"
// steps 1-3; Phobos `@tensorcore`: an i8 dot takes the integer tensor cores
// whenever its shape allows, "When it declines"), on CDNA4's
// v_mfma_i32_32x32x32_i8:
//
//  * 128x128 output tile per workgroup, 4 waves (2x2) of 64x64 outputs, each a
//    2x2 block of 32x32x32 atoms (16 int32 accumulators per lane per atom);
//  * K steps of 128 int8 values: one LDS row per M (or N) index holds 128
//    bytes, eight 16-byte chunks, chunk c of row r at c ^ ((r ^ (r>>3)) & 7)
//    (the 16-bit kernels' layout, in bytes); an atom fragment is 16
//    consecutive K-values of one row (lanes 0-31 the first 16 of the atom's
//    32, lanes 32-63 the second), one ds_read_b128;
//  * global -> VGPR -> LDS staging, two LDS stages, the next K step loaded
//    while the current one is multiplied. K-contiguous operands move in
//    16-byte pieces when the piece is whole and aligned, bytewise otherwise;
//    M/N-contiguous operands are read 16 values along M (or N) and written
//    into their K-contiguous LDS rows byte by byte;
//  * out-of-range elements are staged as zeros (their products are zero), C
//    loads and D stores are predicated.
#include "common.h"

#include <cstdint>

namespace dgt {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 128, kThreads = 256;
constexpr int kTM = 2, kTN = 2;           // atoms per wave
constexpr int kBox = kBM * kBK;           // bytes of one operand box (BM == BN)
constexpr int kStage = 2 * kBox;
constexpr int kPieces = kBox / 16 / kThreads;  // 16-byte pieces per thread per operand: 4

__device__ inline int i8_lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// One operand's 128 x 128 box (rows: M or N indices; K) at (r0, k0).
// KCONTIG: element (r, k) is X[r * ld + k]; otherwise X[k * ld + r].
template <bool KCONTIG>
struct I8Stager {
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
        *reinterpret_cast<u32x4_t*>(lds + i8_lds_off(id >> 3, id & 7)) = v[i];
      } else {
        // byte q of the piece is element (row 16 * (id % 8) + q, K id / 8)
        const int kk = id >> 3, rb = (id & 7) << 4;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const uint8_t b = (uint8_t)(v[i][q >> 2] >> (8 * (q & 3)));
          lds[i8_lds_off(rb + q, kk >> 4) + (kk & 15)] = (char)b;
        }
      }
    }
  }
};

struct I8Frags {
  i32x4 a[kTM], b[kTN];
};

__device__ inline void i8_read(I8Frags& f, const char* As, const char* Bs, int a_row0, int b_row0,
                               int chunk) {
#pragma unroll
  for (int i = 0; i < kTM; ++i)
    f.a[i] = *reinterpret_cast<const i32x4*>(As + i8_lds_off(a_row0 + 32 * i, chunk));
#pragma unroll
  for (int j = 0; j < kTN; ++j)
    f.b[j] = *reinterpret_cast<const i32x4*>(Bs + i8_lds_off(b_row0 + 32 * j, chunk));
}

template <bool TA, bool TB>
__global__ void __launch_bounds__(kThreads) gemm_i8_kernel(const GemmI8Args p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  I8Stager<!TA> sa;  // A is K-contiguous unless transposed
  I8Stager<TB> sb;   // B is K-contiguous only when transposed
  i32x16 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  const int KT = (p.K + kBK - 1) / kBK;
  const int a_row0 = wm * 64 + (lane & 31), b_row0 = wn * 64 + (lane & 31);
  const int half = lane >> 5;  // which 16 K-values of a 32-deep atom

  if (KT > 0) {
    sa.load(p.A, p.lda, m0, p.M, 0, p.K, tid, p.a_vec16);
    sb.load(p.B, p.ldb, n0, p.N, 0, p.K, tid, p.b_vec16);
    sa.store(smem, tid);
    sb.store(smem + kBox, tid);
    __syncthreads();
  }
  for (int kt = 0; kt < KT; ++kt) {
    const char* As = smem + (kt & 1) * kStage;
    const char* Bs = As + kBox;
    if (kt + 1 < KT) {
      sa.load(p.A, p.lda, m0, p.M, (kt + 1) * kBK, p.K, tid, p.a_vec16);
      sb.load(p.B, p.ldb, n0, p.N, (kt + 1) * kBK, p.K, tid, p.b_vec16);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      I8Frags f;
      i8_read(f, As, Bs, a_row0, b_row0, 2 * ks + half);
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      char* nA = smem + ((kt + 1) & 1) * kStage;
      sa.store(nA, tid);
      sb.store(nA + kBox, tid);
    }
    __syncthreads();
  }

  // Epilogue: accumulator v of lane l in atom (i, j) is row 8*(v/4) + 4*(l/32)
  // + v%4, column l%32 of the atom; int32 arithmetic wraps (done unsigned).
  const unsigned alpha = (unsigned)p.alpha, beta = (unsigned)p.beta;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm * 64 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int c = n0 + wn * 64 + 32 * j + (lane & 31);
        if (r < p.M && c < p.N) {
          unsigned d = alpha * (unsigned)acc[i][j][v];
          if (p.read_c) d += beta * (unsigned)p.C[(int64_t)r * p.ldc + c];
          p.D[(int64_t)r * p.ldd + c] = (int)d;
        }
      }
}

}  // namespace

hipError_t launch_i8(bool ta, bool tb, const GemmI8Args& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(kThreads);
  if (!ta && tb) gemm_i8_kernel<false, true><<<grid, block, 0, s>>>(a);
  else if (!ta && !tb) gemm_i8_kernel<false, false><<<grid, block, 0, s>>>(a);
  else if (ta && tb) gemm_i8_kernel<true, true><<<grid, block, 0, s>>>(a);
  else gemm_i8_kernel<true, false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

int i8_tile_m() { return kBM; }
int i8_tile_n() { return kBN; }

}  // namespace dgt
