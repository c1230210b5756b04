/*
 * dense_gemm_tile.h -- C ABI of the MI355X (gfx950) dense GEMM library
 * (libdense_gemm_tile_amd.so).
 *
 * Operation (all matrices row-major):
 *
 *   D = alpha * op(A) @ op(B) + beta * C
 *
 *   op(A)[i,k] = transA ? A[k*lda + i] : A[i*lda + k]      (op(A) is M x K)
 *   op(B)[k,j] = transB ? B[j*ldb + k] : B[k*ldb + j]      (op(B) is K x N)
 *   C[i,j] = C[i*ldc + j],  D[i,j] = D[i*ldd + j]           (M x N, float32)
 *
 * This is the contraction of the TIRx `gemm` tile primitive (Apache TVM docs,
 * TIRx tile primitives, `gemm`: opening paragraph), with A and B f16 or bf16
 * and a float32 accumulator ("What it accepts", dtype row). The transpose flags
 * describe only the stored orientation ("Algorithm" step 1). alpha and beta are
 * general float32 scalars as in the Phobos gemm example's epilogue (Phobos docs,
 * `@tensorcore`, the sm_75/sm_80 kernel pair); beta == 0 means C is not read and
 * D starts from zero (TVM `gemm`, "How inputs change the algorithm", beta row).
 * D may be the same buffer as C (the in-place accumulate form, as the TVM demo
 * passes its D fragment as C, and the Phobos kernel stores back into C).
 *
 * Shapes that do not tile the matrix-core atom are not an error: they run on a
 * masked matrix-core path or on a VALU-FMA fallback with the same result up to
 * rounding (Phobos `@tensorcore`, "When it declines"). gemm_last_path() names
 * the path taken and, for the fallback, why.
 *
 * Pointers: A, B, C, D are DEVICE pointers owned by the caller. The library
 * allocates, frees and synchronises nothing. Work is enqueued on `stream`
 * (a hipStream_t; NULL means the default stream) and gemm() returns before it
 * completes. Error and path strings are thread-local; concurrent calls on
 * different threads are safe. A call enqueues kernel launches only (no
 * memset, copy or event), so calls on a stream under capture are recorded
 * into the HIP graph and replay like the eager calls.
 */
#ifndef DENSE_GEMM_TILE_H
#define DENSE_GEMM_TILE_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define GEMM_API __attribute__((visibility("default")))
#else
#define GEMM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. Any non-zero return launches nothing (except GEMM_ERR_HIP,
 * which reports a failed launch) and sets gemm_last_error(). */
#define GEMM_OK 0
#define GEMM_ERR_INVALID_ARG 1 /* negative dim, ld too small, NULL or misaligned pointer */
#define GEMM_ERR_UNSUPPORTED 2 /* dtype code not 0..5, or a forced path that cannot run */
#define GEMM_ERR_ALIAS 3       /* D overlaps A or B, or overlaps C other than exactly */
#define GEMM_ERR_HIP 4         /* a HIP runtime call failed; message has its text */

/* Operand dtype codes (A and B share one; C and D are always float32). */
#define GEMM_DTYPE_F16 0
#define GEMM_DTYPE_BF16 1
/* A and B hold float32 values that are rounded to f16 / bf16 (to nearest,
 * ties to even) as they are staged; the product then runs on the f16 / bf16
 * matrix cores with the float32 accumulator (Phobos @tensorcore, "The forms":
 * float32 tensors traded to 16-bit inputs for matrix-core speed). Leading
 * dimensions still count elements (now 4 bytes each). */
#define GEMM_DTYPE_F32_F16 2
#define GEMM_DTYPE_F32_BF16 3
/* A and B hold 8-bit float codes, OCP E4M3 (bias 7, no infinity, max 448) or
 * E5M2 (bias 15, IEEE-style specials), multiplied on the 8-bit float matrix
 * cores with the float32 accumulator and unit block scales: the fp8
 * precision of the gemm_async variants (TVM gemm, restated: the precision
 * list). Leading dimensions count bytes; any alignment. */
#define GEMM_DTYPE_F8_E4M3 4
#define GEMM_DTYPE_F8_E5M2 5

/*
 * gemm: enqueue D = alpha*op(A)@op(B) + beta*C on `stream`.
 *
 * M, N, K   >= 0. M == 0 or N == 0: nothing to do, returns GEMM_OK.
 *           K == 0 or alpha == 0: D = beta*C (A and B are not read).
 * dtype     GEMM_DTYPE_F16 or GEMM_DTYPE_BF16, the element type of A and B;
 *           or GEMM_DTYPE_F32_F16 / GEMM_DTYPE_F32_BF16 for float32 A and B
 *           rounded to f16 / bf16 while staged; or GEMM_DTYPE_F8_E4M3 /
 *           GEMM_DTYPE_F8_E5M2 for 8-bit float codes (matrix-core paths only:
 *           GEMM_FORCE_PATH=fma returns GEMM_ERR_UNSUPPORTED for 2..5).
 * transA/B  0 or 1 (any non-zero means 1). transA: A is stored [K][M];
 *           transB: B is stored [N][K].
 * lda       >= max(1, transA ? M : K), in elements; ldb >= max(1, transB ? K : N);
 *           ldd >= max(1, N); ldc >= max(1, N) when beta != 0.
 * A, B      device pointers, 2-byte aligned (4-byte for float32 operands, any
 *           for 8-bit codes); may be NULL only when K == 0 or alpha == 0.
 * C         device float32 pointer, 4-byte aligned; ignored (may be NULL)
 *           when beta == 0.
 * D         device float32 pointer, 4-byte aligned.
 * Aliasing  D must not overlap A or B. D may equal C exactly (same pointer and
 *           ldc == ldd); any other overlap of C and D is rejected.
 * stream    hipStream_t cast to void*.
 *
 * Path: every call runs on the matrix cores. An operand whose base address or
 * row pitch is not a multiple of 16 bytes is staged through registers with
 * dword-aligned loads (or, on the small-tile kernels, read with the widest
 * loads both allow); slower, same result up to rounding order. A call just
 * past a multiple of the 256x256 tile may run as three launches (whole
 * tiles, remainder rows, remainder columns); each element of D is still
 * computed once. The VALU FMA path computes the same contraction with f32
 * FMAs and runs only when forced.
 *
 * Environment: GEMM_LOG=debug prints one line per call to stderr (path, tile,
 * reason); GEMM_FORCE_PATH=mfma|fma forces the matrix-core or the VALU path;
 * GEMM_FORCE_TILE=<tile name> picks a matrix-core tile configuration;
 * GEMM_RING_MODE=shared|ksplit2|deep|pp|ppdeep picks the form of the 128x128
 * kernel; GEMM_STAGE_DEPTH=1|2 sets how far ahead a single staged operand is
 * requested. Any forcing switch also keeps a call in one launch.
 */
GEMM_API int gemm(int64_t M, int64_t N, int64_t K, int dtype, int transA, int transB,
         float alpha, float beta,
         const void* A, int64_t lda, const void* B, int64_t ldb,
         const float* C, int64_t ldc, float* D, int64_t ldd, void* stream);

/*
 * gemm_validate: the host-side part of gemm() without any launch and without
 * touching a GPU: argument checks, then path and tile selection. Returns the
 * status gemm() would return before launching, and records the chosen path in
 * gemm_last_path(). Pointers are only compared, never dereferenced.
 */
GEMM_API int gemm_validate(int64_t M, int64_t N, int64_t K, int dtype, int transA, int transB,
                  float alpha, float beta,
                  const void* A, int64_t lda, const void* B, int64_t ldb,
                  const float* C, int64_t ldc, const float* D, int64_t ldd);

/* Message for the last non-zero return on this thread ("" if none). The
 * pointer stays valid until the next call on this thread. */
GEMM_API const char* gemm_last_error(void);

/* Path of the last gemm()/gemm_validate() on this thread, e.g.
 * "mfma t256x256x64 w2x4 a32x32x16 NT epi=beta0 pingpong",
 * "mfma t256x256x64 w2x4 a32x32x16 NT epi=beta0 pingpong f32->bf16" (float32
 * operands rounded as their fragments are read),
 * "mfma t32x32x64k4 w1x1 a32x32x16 NN epi=general ksplit4" (K split over four
 * wave groups of one workgroup, for grids with few output tiles),
 * "mfma t128x128x64 w2x2 a32x32x16 TN epi=general masked narrow staging
 * (A: 2-byte loads, row pitch 8194 B is not a multiple of 16 B)",
 * "fp8 e4m3 mfma t256x256x128 w2x4 a32x32x64 NT epi=beta0 pingpong" or
 * "fma t64x64x16 NN epi=beta0: forced by GEMM_FORCE_PATH=fma". Same lifetime
 * as above. */
GEMM_API const char* gemm_last_path(void);

/*
 * gemm_i8: enqueue D = alpha*op(A)@op(B) + beta*C for int8 A and B with an
 * int32 accumulator and int32 C and D: the integer tensor-core form of the
 * same contraction (Phobos @tensorcore, "When it declines": an i8 dot takes
 * the integer tensor cores whenever its shape allows). Every sum, and the
 * epilogue, wraps modulo 2^32 like int32 arithmetic.
 *
 * Arguments as for gemm(), with: alpha, beta int32; A, B int8 device pointers
 * (any alignment; leading dimensions in bytes = elements); C, D int32 device
 * pointers, 4-byte aligned. beta == 0: C is not read (may be NULL). K == 0 or
 * alpha == 0: D = beta*C (A and B are not read). M == 0 or N == 0: nothing
 * to do. D may equal C exactly; it must not overlap A or B. Same return
 * codes, thread-local error/path strings and GEMM_LOG=debug line as gemm().
 */
GEMM_API int gemm_i8(int64_t M, int64_t N, int64_t K, int transA, int transB, int32_t alpha,
            int32_t beta, const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
            const int32_t* C, int64_t ldc, int32_t* D, int64_t ldd, void* stream);

/* gemm_i8_validate: the host-side checks of gemm_i8() without any launch. */
GEMM_API int gemm_i8_validate(int64_t M, int64_t N, int64_t K, int transA, int transB,
            int32_t alpha, int32_t beta, const int8_t* A, int64_t lda, const int8_t* B,
            int64_t ldb, const int32_t* C, int64_t ldc, const int32_t* D, int64_t ldd);

/*
 * gemm_tile_order: the output-tile scheduler's workgroup -> tile map, computed
 * on the host (the kernels use the same function). For tiles_m x tiles_n tiles
 * it writes, for each workgroup id w in [0, tiles_m*tiles_n), the tile row
 * tm[w] and column tn[w]. tm and tn are host arrays of tiles_m*tiles_n int32.
 * group_m is the tile-row group height of the grouped order (>= 1).
 * Returns GEMM_OK or GEMM_ERR_INVALID_ARG.
 */
GEMM_API int gemm_tile_order(int64_t tiles_m, int64_t tiles_n, int group_m, int32_t* tm, int32_t* tn);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_TILE_H */
