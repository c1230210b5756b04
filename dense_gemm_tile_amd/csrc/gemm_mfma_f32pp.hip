// Whole 256x256 tiles of float32 operands, both K-contiguous (A stored [M][K],
// B stored [N][K]), on the two-group direct-to-LDS design of the 16-bit
// kernel. The operands reach LDS as float32 and are rounded to f16 or bf16
// (nearest, ties to even) in registers as each fragment is read, so an f32
// call moves no more than its own operand bytes through HBM and the matrix
// cores see the same 16-bit values as when the caller rounds beforehand
// (Phobos @tensorcore, "The forms": f32 tensors on the tensor cores trade
// input precision for speed).
//
// A 128-byte row slice holds 32 K-values here, so a K slice is 32 deep: two
// MFMA sub-steps (16 MFMAs per wave) per compute phase against the same 32 KiB
// half slice of loads per memory phase as the 16-bit kernel. Ring, slots,
// phases, waits and barriers are the 16-bit kernel's.
#include "gemm_mfma_pingpong.h"

namespace dgt {

namespace {

typedef float pp_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 pp_bf2 __attribute__((ext_vector_type(2)));
typedef _Float16 pp_h2 __attribute__((ext_vector_type(2)));

// Two floats -> one dword of two 16-bit values (first in the low half), round
// to nearest even: v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32.
__device__ __forceinline__ unsigned cvt_pk(TagBF16, float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(pp_f2{lo, hi}, pp_bf2));
}
__device__ __forceinline__ unsigned cvt_pk(TagF16, float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(pp_f2{lo, hi}, pp_h2));
}

// Lane l's fragment of one atom in sub-step ks: 8 consecutive K-values of
// one row at K = 16*ks + 8*(l >> 5), i.e. 32 bytes = chunks 4ks + 2(l >> 5)
// and the next one. `off` is the byte offset of chunk 2(l >> 5) of the row in
// the slot; the row's swizzle XORs the chunk index, so chunk bit 2 (ks) and
// bit 0 (second half) are XOR-ed into the offset.
template <class Tag>
__device__ __forceinline__ u32x4 read_f32_frag(const char* slot, int off, int ks) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(slot + (off ^ (ks << 6)));
  const f32x4 hi = *reinterpret_cast<const f32x4*>(slot + (off ^ (ks << 6) ^ 16));
  return u32x4{cvt_pk(Tag{}, lo[0], lo[1]), cvt_pk(Tag{}, lo[2], lo[3]),
               cvt_pk(Tag{}, hi[0], hi[1]), cvt_pk(Tag{}, hi[2], hi[3])};
}

template <class Tag, int EPI>
__global__ void __launch_bounds__(PingPongCfg::THREADS) gemm_pp_f32_kernel(const GemmArgs p) {
  using C = PingPongCfg;
  using At = typename C::At;
  using acc_t = typename At::acc_t;
  constexpr int KSL = 32;          // K-values per slice (128 bytes of float32)
  constexpr int KS = KSL / At::K;  // MFMA sub-steps per slice
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: no divergent barriers
  const int group = wave >> 2, lw = wave & 3;
  const int wm = group, wn = lw;
  int tm, tn;
  schedule_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  PpOperand<false, C::TM> a;
  PpOperand<false, C::TN> b;
  a.init_load(p.A, p.lda, m0, lw, lane, 4);
  b.init_load(p.B, p.ldb, n0, lw, lane, 4);
  int offA[C::TM], offB[C::TN];  // fragment offsets within a slot, sub-step 0
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
    offA[i] = PpOperand<false, C::TM>::lds_off(wm * C::WTM + 32 * i + (lane & 31), 2 * (lane >> 5));
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
    offB[j] = PpOperand<false, C::TN>::lds_off(wn * C::WTN + 32 * j + (lane & 31), 2 * (lane >> 5));

  acc_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < At::NACC; ++v) acc[i][j][v] = 0.0f;

  auto issue_a = [&](int slice, int slot) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) a.issue(smem + slot * C::SLOT_BYTES, lw, i, slice);
  };
  auto issue_b = [&](int slice, int slot) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) b.issue(smem + slot * C::SLOT_BYTES, lw, i, slice);
  };

  // Phases as in the 16-bit kernel: group 0 reads slice s in phase 2s+1 and
  // multiplies it in 2s+2, group 1 one phase later; A of slice t in slot
  // 2t % 5 (loaded by group 1), B in slot (2t+1) % 5 (loaded by group 0).
  const int KT = p.K / KSL;
  if (group == 1) {
    issue_a(0, 0);
    if (KT > 1) {
      issue_a(1, 2);
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
    pp_wait_vm<0>();  // A of slice 1, read from phase 3 on
    pp_barrier();
  }
  u32x4 fa[KS][C::TM], fb[KS][C::TN];
  int h = 0;  // (2s) % 5: the slot of A of slice s
  for (int s = 0; s < KT; ++s) {
    asm volatile("" : "+v"(a.row), "+v"(a.c0), "+v"(b.row), "+v"(b.c0));
    asm volatile("" : "+v"(offA[0]), "+v"(offA[1]), "+v"(offA[2]), "+v"(offA[3]),
                 "+v"(offB[0]), "+v"(offB[1]));
    const int sa = h, sb = h == 4 ? 0 : h + 1;
    const char* pa = smem + sa * C::SLOT_BYTES;
    const char* pb = smem + sb * C::SLOT_BYTES;
    // Memory phase: fragments (read and rounded), then this group's half slice.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) fa[ks][i] = read_f32_frag<Tag>(pa, offA[i], ks);
#pragma unroll
      for (int j = 0; j < C::TN; ++j) fb[ks][j] = read_f32_frag<Tag>(pb, offB[j], ks);
    }
    if (group == 0) {
      if (s + 1 < KT) issue_b(s + 1, h >= 2 ? h - 2 : h + 3);  // B of s+1: (2s+3) % 5
      pp_wait_lgkm0();
    } else {
      const bool ld = s + 2 < KT;
      if (ld) issue_a(s + 2, h >= 1 ? h - 1 : h + 4);  // A of s+2: (2s+4) % 5
      if (ld) pp_wait_vm_lgkm0<C::LOADS>();
      else pp_wait_vm_lgkm0<0>();
    }
    pp_barrier();
    // Compute phase.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = At::mma(Tag{}, fa[ks][i], fb[ks][j], acc[i][j]);
    if (group == 0) pp_wait_vm<0>();  // B of slice s+1, read from the next phase on
    pp_barrier();
    h = h >= 3 ? h - 3 : h + 2;
  }
  if (group == 0) pp_barrier();  // matches group 1's idle phase: same barrier count

  store_tile<C, EPI, false>(acc, p, m0 + wm * C::WTM, n0 + wn * C::WTN, lane);
}

template <class Tag>
hipError_t launch_tag(const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(PingPongCfg::THREADS);
  if (a.epi == EPI_BETA0) return launch_kernel(gemm_pp_f32_kernel<Tag, EPI_BETA0>, grid, block, s, a);
  if (a.epi == EPI_ACC_PLUS_C)
    return launch_kernel(gemm_pp_f32_kernel<Tag, EPI_ACC_PLUS_C>, grid, block, s, a);
  return launch_kernel(gemm_pp_f32_kernel<Tag, EPI_GENERAL>, grid, block, s, a);
}

}  // namespace

hipError_t launch_pp_f32(int dtype16, const GemmArgs& a, hipStream_t s) {
  if (dtype16 == 0) return launch_tag<TagF16>(a, s);
  return launch_tag<TagBF16>(a, s);
}

int pp_f32_slice() { return 32; }

}  // namespace dgt
