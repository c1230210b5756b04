// VALU-FMA fallback GEMM and the epilogue-only kernel.
//
// The fallback computes the same contraction with float32 FMAs for shapes and
// layouts the matrix-core staging declines (operand rows that are not 16-byte
// aligned), or when forced. Declining is not an error and the result is the
// same up to rounding (Phobos `@tensorcore`, "When it declines").
//
// Design: 64x64 output tile per 256-thread workgroup, 16-deep K slices staged
// through LDS as float32 (each 16-bit operand element is widened exactly on
// the way in, with any alignment: plain 2-byte loads), 4x4 outputs per thread
// accumulated with fmaf in K order, then the same alpha/beta epilogue as the
// matrix-core path.
#include "common.h"

namespace dgt {

namespace {

__device__ inline float widen(uint16_t h, int dtype) {
  if (dtype == 0) return (float)__builtin_bit_cast(_Float16, h);
  return __builtin_bit_cast(float, (unsigned)h << 16);
}

constexpr int FB_BM = kFmaTileM, FB_BN = kFmaTileN, FB_BK = 16, FB_THREADS = 256;

template <bool TA, bool TB>
__global__ void __launch_bounds__(FB_THREADS) gemm_fma_kernel(const GemmArgs p, int dtype) {
  __shared__ float As[FB_BK][FB_BM];  // As[k][m]
  __shared__ float Bs[FB_BK][FB_BN];  // Bs[k][n]
  const int tid = threadIdx.x;
  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * FB_BM, n0 = tn * FB_BN;
  const int tx = tid % 16, ty = tid / 16;
  const uint16_t* A = static_cast<const uint16_t*>(p.A);
  const uint16_t* B = static_cast<const uint16_t*>(p.B);

  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;

  for (int k0 = 0; k0 < p.K; k0 += FB_BK) {
#pragma unroll
    for (int i = 0; i < (FB_BM * FB_BK) / FB_THREADS; ++i) {
      const int id = tid + i * FB_THREADS;
      // consecutive threads walk the contiguous direction of the stored A
      const int m = TA ? id % FB_BM : id / FB_BK;
      const int k = TA ? id / FB_BM : id % FB_BK;
      const int gm = m0 + m, gk = k0 + k;
      float x = 0.0f;
      if (gm < p.M && gk < p.K)
        x = widen(TA ? A[(int64_t)gk * p.lda + gm] : A[(int64_t)gm * p.lda + gk], dtype);
      As[k][m] = x;
    }
#pragma unroll
    for (int i = 0; i < (FB_BN * FB_BK) / FB_THREADS; ++i) {
      const int id = tid + i * FB_THREADS;
      const int n = TB ? id / FB_BK : id % FB_BN;
      const int k = TB ? id % FB_BK : id / FB_BN;
      const int gn = n0 + n, gk = k0 + k;
      float x = 0.0f;
      if (gn < p.N && gk < p.K)
        x = widen(TB ? B[(int64_t)gn * p.ldb + gk] : B[(int64_t)gk * p.ldb + gn], dtype);
      Bs[k][n] = x;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FB_BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = As[k][ty * 4 + r];
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] = Bs[k][tx * 4 + c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(a[r], b[c], acc[r][c]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gm = m0 + ty * 4 + r;
    if (gm >= p.M) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int gn = n0 + tx * 4 + c;
      if (gn >= p.N) continue;
      const float x = acc[r][c];
      float* dp = p.D + (int64_t)gm * p.ldd + gn;
      if (p.epi == EPI_BETA0) {
        *dp = p.alpha * x;
      } else {
        const float cv = p.C[(int64_t)gm * p.ldc + gn];
        *dp = (p.epi == EPI_ACC_PLUS_C) ? (x + cv) : __builtin_fmaf(p.beta, cv, p.alpha * x);
      }
    }
  }
}

// D = beta*C (K == 0 or alpha == 0). beta == 0 writes zeros without reading C.
__global__ void __launch_bounds__(256) scale_c_kernel(const GemmArgs p) {
  const int64_t total = (int64_t)p.M * p.N;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / p.N, j = e % p.N;
    p.D[i * p.ldd + j] = (p.beta == 0.0f) ? 0.0f : p.beta * p.C[i * p.ldc + j];
  }
}

}  // namespace

hipError_t launch_fma(int dtype, bool ta, bool tb, const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(FB_THREADS);
  if (!ta && !tb) return launch_kernel(gemm_fma_kernel<false, false>, grid, block, s, a, dtype);
  if (!ta && tb) return launch_kernel(gemm_fma_kernel<false, true>, grid, block, s, a, dtype);
  if (ta && !tb) return launch_kernel(gemm_fma_kernel<true, false>, grid, block, s, a, dtype);
  return launch_kernel(gemm_fma_kernel<true, true>, grid, block, s, a, dtype);
}

hipError_t launch_scale_c(const GemmArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.M * a.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return launch_kernel(scale_c_kernel, dim3((unsigned)blocks), dim3(256), s, a);
}

}  // namespace dgt
