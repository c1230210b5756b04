// 256x256 tiles of float32 operands, in any of the four layouts, on the
// two-group direct-to-LDS design of the 16-bit kernel: whole tiles, or edge
// tiles (MASK) when each operand's contiguous dimension is a multiple of 4
// (whole 16-byte pieces; pieces past the operand read as zeros, as there). The operands reach
// LDS as float32 and are rounded to f16 or bf16
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
//
// An M/N-contiguous operand (A stored [K][M], B stored [K][N]) fills a slot
// as the slice's 32 K-rows of 256 values (1 KiB each); 16-byte chunk c of
// row r sits at position c ^ (8 * r3) (r3: bit 3 of r). A load instruction
// of wave lw covers one row (8 lw + i), lane l filling position l. A lane's
// fragment (8 consecutive K of one column) is 8 ds_read_b32 down the rows,
// 1 KiB apart; lanes 0-31 read 32 consecutive columns of one row and lanes
// 32-63 the same columns 8 rows down, which the swizzle moves to the other
// half of the banks.
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

// An M/N-contiguous float32 operand of the two-group kernel (see above).
template <bool MASK>
struct PpF32MN {
  const float* base;  // tile's first column (M or N index), K = 0
  int64_t ld;         // row pitch in elements
  int voff;           // this lane's byte offset within the wave's first row
  int cin, krem0;     // (MASK) this lane's piece starts inside the operand; K - 8 lw
  int klim, crem;     //    K; columns left from the tile's first
  __device__ inline void init_load(const void* X, int64_t ld_, int c0, int lw, int lane) {
    base = static_cast<const float*>(X) + c0;
    ld = ld_;
    // rows 8 lw .. 8 lw + 7 all have r3 = lw & 1
    voff = (int)((int64_t)(8 * lw) * ld * 4) + ((lane ^ (8 * (lw & 1))) << 4);
  }
  // (MASK) the operand's extent from this tile: clim columns (M or N), K.
  __device__ inline void set_limits(int c0, int clim, int K, int lw, int lane) {
    crem = clim - c0;
    cin = 4 * (lane ^ (8 * (lw & 1))) < crem;
    krem0 = K - 8 * lw;
    klim = K;
  }
  __device__ __forceinline__ void issue(char* slot, int lw, int i, int slice) const {
    // The slice's first K row is folded into the resource base, so the
    // 32-bit offsets stay within its 32 rows.
    const float* b = base + (int64_t)slice * 32 * ld;
    if constexpr (!MASK) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(b), (pp_lds_ptr_t)(slot + (lw * 8 + i) * 1024),
                                               16, voff, (int)(i * ld * 4), 0, 0);
    } else {
      // This instruction's K row is slice*32 + 8 lw + i; the record count
      // ends at the last K row's last valid column, counted from b.
      const int64_t n = 4 * ((int64_t)(klim - 1 - slice * 32) * ld + crem);
      const unsigned nrec = n <= 0 ? 0u : (n > 0x7FFFFFFC ? 0x7FFFFFFCu : (unsigned)n);
      const int voffm = (cin && krem0 - slice * 32 - i > 0) ? voff + (int)(i * ld * 4) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc_n(b, nrec),
                                               (pp_lds_ptr_t)(slot + (lw * 8 + i) * 1024), 16, voffm,
                                               0, 0, 0);
    }
  }
  // Sub-step-0 byte offset of lane l's fragment of the 32x32 atom whose
  // first column is col0 (within the tile): column col0 + l%32, rows
  // 8 (l/32) .. +7.
  __device__ static inline int frag_off(int col0, int lane) {
    const int col = col0 + (lane & 31), h = lane >> 5;
    return (8 * h) * 1024 + (((col >> 2) ^ (8 * h)) << 4) + ((col & 3) << 2);
  }
};

// Lane l's fragment of an M/N-contiguous operand in sub-step ks (rows 16 ks
// + 8 (l/32) .. +7 of its column), rounded to Tag's type.
template <class Tag>
__device__ __forceinline__ u32x4 read_f32_frag_mn(const char* slot, int off, int ks) {
  const float* q = reinterpret_cast<const float*>(slot + off + ks * 16 * 1024);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = q[e * 256];
  return u32x4{cvt_pk(Tag{}, v[0], v[1]), cvt_pk(Tag{}, v[2], v[3]), cvt_pk(Tag{}, v[4], v[5]),
               cvt_pk(Tag{}, v[6], v[7])};
}

template <bool MN, int NFRAG, bool MASK>
struct PpF32Op {
  using type = PpOperand<false, NFRAG, 32, MASK>;
};
template <int NFRAG, bool MASK>
struct PpF32Op<true, NFRAG, MASK> {
  using type = PpF32MN<MASK>;
};

template <class Tag, int EPI, bool AMN, bool BMN, bool MASK>
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

  typename PpF32Op<AMN, C::TM, MASK>::type a;
  typename PpF32Op<BMN, C::TN, MASK>::type b;
  if constexpr (AMN) a.init_load(p.A, p.lda, m0, lw, lane);
  else a.init_load(p.A, p.lda, m0, lw, lane, 4);
  if constexpr (BMN) b.init_load(p.B, p.ldb, n0, lw, lane);
  else b.init_load(p.B, p.ldb, n0, lw, lane, 4);
  if constexpr (MASK) {
    if constexpr (AMN) a.set_limits(m0, p.M, p.K, lw, lane);
    else a.set_limits(m0, p.M, 4 * p.K, lw, lane);
    if constexpr (BMN) b.set_limits(n0, p.N, p.K, lw, lane);
    else b.set_limits(n0, p.N, 4 * p.K, lw, lane);
  }
  int offA[C::TM], offB[C::TN];  // fragment offsets within a slot, sub-step 0
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
    offA[i] = AMN ? PpF32MN<MASK>::frag_off(wm * C::WTM + 32 * i, lane)
                  : PpOperand<false, C::TM>::lds_off(wm * C::WTM + 32 * i + (lane & 31),
                                                     2 * (lane >> 5));
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
    offB[j] = BMN ? PpF32MN<MASK>::frag_off(wn * C::WTN + 32 * j, lane)
                  : PpOperand<false, C::TN>::lds_off(wn * C::WTN + 32 * j + (lane & 31),
                                                     2 * (lane >> 5));

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
  // Slices: whole ones, or (edge tiles) the last one cut short and zero-filled.
  const int KT = MASK ? (p.K + KSL - 1) / KSL : p.K / KSL;
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
    if constexpr (AMN) asm volatile("" : "+v"(a.voff));
    else asm volatile("" : "+v"(a.row), "+v"(a.c0));
    if constexpr (BMN) asm volatile("" : "+v"(b.voff));
    else asm volatile("" : "+v"(b.row), "+v"(b.c0));
    if constexpr (MASK) {
      if constexpr (AMN) asm volatile("" : "+v"(a.cin), "+v"(a.krem0));
      else asm volatile("" : "+v"(a.rmask));
      if constexpr (BMN) asm volatile("" : "+v"(b.cin), "+v"(b.krem0));
      else asm volatile("" : "+v"(b.rmask));
    }
    asm volatile("" : "+v"(offA[0]), "+v"(offA[1]), "+v"(offA[2]), "+v"(offA[3]),
                 "+v"(offB[0]), "+v"(offB[1]));
    const int sa = h, sb = h == 4 ? 0 : h + 1;
    const char* pa = smem + sa * C::SLOT_BYTES;
    const char* pb = smem + sb * C::SLOT_BYTES;
    // Memory phase: fragments (read and rounded), then this group's half slice.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        fa[ks][i] = AMN ? read_f32_frag_mn<Tag>(pa, offA[i], ks) : read_f32_frag<Tag>(pa, offA[i], ks);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        fb[ks][j] = BMN ? read_f32_frag_mn<Tag>(pb, offB[j], ks) : read_f32_frag<Tag>(pb, offB[j], ks);
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

  store_tile<C, EPI, MASK>(acc, p, m0 + wm * C::WTM, n0 + wn * C::WTN, lane);
}

template <class Tag, bool AMN, bool BMN, bool MASK>
hipError_t launch_layout(const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(PingPongCfg::THREADS);
  if (a.epi == EPI_BETA0)
    return launch_kernel(gemm_pp_f32_kernel<Tag, EPI_BETA0, AMN, BMN, MASK>, grid, block, s, a);
  if (a.epi == EPI_ACC_PLUS_C)
    return launch_kernel(gemm_pp_f32_kernel<Tag, EPI_ACC_PLUS_C, AMN, BMN, MASK>, grid, block, s,
                         a);
  return launch_kernel(gemm_pp_f32_kernel<Tag, EPI_GENERAL, AMN, BMN, MASK>, grid, block, s, a);
}

template <class Tag, bool MASK>
hipError_t launch_tag(bool ta, bool tb, const GemmArgs& a, hipStream_t s) {
  // A is M-contiguous when stored transposed; B is N-contiguous when not.
  if (!ta && tb) return launch_layout<Tag, false, false, MASK>(a, s);
  if (!ta && !tb) return launch_layout<Tag, false, true, MASK>(a, s);
  if (ta && tb) return launch_layout<Tag, true, false, MASK>(a, s);
  return launch_layout<Tag, true, true, MASK>(a, s);
}

}  // namespace

hipError_t launch_pp_f32(int dtype16, bool ta, bool tb, bool masked, const GemmArgs& a,
                         hipStream_t s) {
  if (masked) {
    if (dtype16 == 0) return launch_tag<TagF16, true>(ta, tb, a, s);
    return launch_tag<TagBF16, true>(ta, tb, a, s);
  }
  if (dtype16 == 0) return launch_tag<TagF16, false>(ta, tb, a, s);
  return launch_tag<TagBF16, false>(ta, tb, a, s);
}

int pp_f32_slice() { return 32; }

}  // namespace dgt
