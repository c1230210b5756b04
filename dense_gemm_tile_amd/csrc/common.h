// Internal declarations shared by the host dispatcher and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgt {

// Everything a kernel needs for one call. Plain values only.
struct GemmArgs {
  const void* A;
  const void* B;
  const float* C;
  float* D;
  int64_t lda, ldb, ldc, ldd;  // leading dimensions, in elements
  int M, N, K;
  float alpha, beta;
  int epi;       // Epilogue kind, see below
  int wide_epi;  // 1: D (and C when read) allow 16-byte accesses (base and
                 //    leading dimension multiples of 16 bytes)
  int tiles_m;   // output tiles along M / N for the tile scheduler
  int tiles_n;
  int group_m;   // tile-row group height of the grouped order
  int a_vw;      // staging vector width of A in 16-bit elements (8, 4, 2 or 1):
  int b_vw;      //    the widest whose byte size divides A's base and row pitch
                 //    (same for B); below 8 only the masked kernel runs
  int src32;     // 0: A and B hold 16-bit values; 1 / 2: A and B hold float32
                 //    values, rounded to f16 / bf16 (nearest, ties to even) as
                 //    they are staged (masked kernel only); a_vw, b_vw then
                 //    count float32 elements (4, 2 or 1)
  int a_fast;    // 1: whole boxes of A may be read without bounds checks
  int b_fast;    //    (16-bit values; 32-bit byte offsets reach every box):
                 //    the masked kernel then reads the whole K steps of its
                 //    interior tiles that way (same for B)
  int a_direct;  // 128x128 ring kernel: 1 if A is loaded straight into LDS
  int b_direct;  //    (16-byte rows, edges of its contiguous dimension on
                 //    multiples of 8 elements), 0 if staged through registers
  int ring_mode; // 128x128 ring kernel: RingMode below
  int stage_depth; // 128x128 ring kernel with exactly one staged 16-bit operand:
                   //    2 requests its loads three slices ahead (two register
                   //    sets), 1 two slices ahead (one set)
  int mfold;     // 128x128 ring kernel (two K groups, 16-bit operands):
                 //    rows M - mfold .. M - 1 (0 < mfold <= 4) lie past the
                 //    tiles_m whole tile rows and are computed by the last of
                 //    them; 0: none
};

// Forms of the 128x128 ring kernel.
enum RingMode : int {
  RING_SHARED = 0,   // five half-slots (80 KiB): two workgroups share a CU
  RING_KSPLIT2 = 1,  // two K groups of 4 waves per workgroup, a ring each
  RING_DEEP = 2,     // ten half-slots (160 KiB), slices requested four ahead;
                     //    both operands loaded straight into LDS
  RING_PP = 3,       // two wave groups taking turns, five half-slots (80 KiB);
                     //    both operands loaded straight into LDS
  RING_PP_DEEP = 4,  // the same with ten half-slots (160 KiB), loads further ahead
};

// Arguments of the 1-byte-operand kernels (see gemm_byte.hip): int8 ->
// int32 (integer alpha/beta, int32 C/D) or 8-bit float -> f32 (f32 alpha/beta
// and C/D).
struct GemmByteArgs {
  const void* A;
  const void* B;
  const void* C;
  void* D;
  int64_t lda, ldb, ldc, ldd;  // in elements
  int M, N, K;
  int alpha_i, beta_i;     // int8 form
  float alpha_f, beta_f;   // 8-bit float form
  int read_c;              // beta != 0
  int a_vec16, b_vec16;    // base and row pitch multiples of 16 bytes
  int cd_vec16;            // D (and C when read): base and row pitch multiples of 16 bytes
  int cd_scalar;           // two-group kernel with edge tiles: C and D accessed element by
                           //    element (D or C rows not 16-byte aligned, or N % 4 != 0)
  int tiles_m, tiles_n, group_m;
  int pingpong;  // the two-group kernel: 1 on whole 256x256 tiles, 2 with edge tiles
};
enum ByteKind : int { BYTE_I8 = 0, BYTE_F8E4M3 = 1, BYTE_F8E5M2 = 2 };

// Epilogue kinds. All three compute alpha*acc + beta*C; the specialised ones
// only skip work whose result is known exactly (C not read when beta == 0,
// multiplies by 1 dropped when alpha == beta == 1).
enum Epilogue : int {
  EPI_BETA0 = 0,      // D = alpha*acc          (C never read)
  EPI_ACC_PLUS_C = 1, // D = acc + C            (alpha == 1, beta == 1)
  EPI_GENERAL = 2,    // D = fma(beta, C, alpha*acc)
};

// Number of XCDs (each with its own L2) on MI355X. Workgroups of one launch are
// handed to XCDs round-robin by workgroup id; the scheduler below regroups ids
// so that tiles which share operand panels land on the same XCD. Any value
// gives a correct (bijective) mapping; 8 is the one that matches the chip.
constexpr int kNumXcd = 8;

// Workgroup id -> logical tile index: XCD x receives ids x, x+8, x+16, ... and
// the remap gives those ids one contiguous range of logical indices.
__host__ __device__ inline int xcd_remap(int bid, int nwg) {
  const int xcd = bid % kNumXcd;
  const int idx = bid / kNumXcd;
  const int q = nwg / kNumXcd;
  const int r = nwg % kNumXcd;
  return xcd * q + (xcd < r ? xcd : r) + idx;
}

// Logical tile index -> (tile row, tile column) in grouped order: walk
// group_m tile rows column by column, so that consecutive indices share the
// A row panels of the group and each B column panel is reused group_m times.
__host__ __device__ inline void grouped_tile(int lid, int tiles_m, int tiles_n, int group_m,
                                             int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int g = lid / per_group;
  const int first_m = g * group_m;
  const int rows_left = tiles_m - first_m;
  const int gsz = rows_left < group_m ? rows_left : group_m;
  const int in = lid - g * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

__host__ __device__ inline void schedule_tile(int bid, int tiles_m, int tiles_n, int group_m,
                                              int& tm, int& tn) {
  const int lid = xcd_remap(bid, tiles_m * tiles_n);
  grouped_tile(lid, tiles_m, tiles_n, group_m, tm, tn);
}

// Enqueue kernel `k` on `s` with the given arguments. The status returned is
// that of this launch alone (hipLaunchKernel), so an error left behind by an
// earlier, unrelated HIP call on the thread is neither reported nor cleared.
template <class T>
struct same_type {
  using type = T;
};
template <class... P>
inline hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s,
                                typename same_type<P>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, s);
}

// Launchers (defined next to their kernels). They return the HIP status of
// the launch.
struct MfmaTileInfo {
  const char* name;
  int bm, bn, bk;
  int waves_m, waves_n;
  int atom_m, atom_n, atom_k;
  int kg;  // K groups: waves split K kg ways within one workgroup
};

// Matrix-core tile configurations, largest first.
enum MfmaTile : int { TILE_256x256 = 0, TILE_128x128 = 1, TILE_64x64 = 2, TILE_16x16 = 3,
                      TILE_32x32K4 = 4, TILE_32x32K8 = 5, TILE_64x64K4 = 6,
                      NUM_MFMA_TILES = 7 };
const MfmaTileInfo& mfma_tile_info(int tile);

hipError_t launch_mfma(int tile, int dtype, bool transA, bool transB, bool masked,
                       const GemmArgs& a, hipStream_t stream);
// 128x128 tiles on the direct-to-LDS ring kernel: f16 (dtype 0) or bf16 (1)
// operands, any layout, any M/N/K, row pitches up to the 32-bit offset rule.
hipError_t launch_ring128(int dtype, bool transA, bool transB, const GemmArgs& a,
                          hipStream_t stream);
// Output tile of the VALU-FMA fallback.
constexpr int kFmaTileM = 64, kFmaTileN = 64;

hipError_t launch_fma(int dtype, bool transA, bool transB, const GemmArgs& a,
                      hipStream_t stream);
hipError_t launch_byte(int kind, bool ta, bool tb, const GemmByteArgs& a, hipStream_t s);
int byte_tile_m();
int byte_tile_n();
int byte_pp_tile();
hipError_t launch_scale_c(const GemmArgs& a, hipStream_t stream);
// 256x256 tiles of float32 A and B (src32 calls, any layout), rounded to
// f16 (dtype16 0) or bf16 (1) as fragments are read: whole tiles with K a
// multiple of pp_f32_slice(), or (masked) edge tiles and K tails when each
// operand's contiguous dimension is a multiple of 4.
hipError_t launch_pp_f32(int dtype16, bool transA, bool transB, bool masked, const GemmArgs& a,
                         hipStream_t stream);
int pp_f32_slice();

}  // namespace dgt
