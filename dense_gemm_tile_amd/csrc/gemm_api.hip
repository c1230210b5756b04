// Host side of the C ABI: argument checks, path and tile selection, launch.
//
// Checks follow the contract of the TIRx `gemm` primitive, which rejects a
// call rather than emit a wrong instruction (TVM TIRx `gemm`: "What it
// accepts"; its Chinese restatement, section 2, lists the rejection reasons and
// the normalisation to A=[M,K], B=[K,N]). Shapes that do not tile the
// matrix-core atom are not rejected: they run masked, or on the VALU fallback,
// and the chosen path and its reason are recorded, like the debug log that
// names each declined dot (Phobos `@tensorcore`, "When it declines").
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "dense_gemm_tile.h"
#include "common.h"

extern char** environ;  // POSIX: the process environment (read by read_env)

namespace dgt {
namespace {

thread_local std::string g_err;
thread_local std::string g_path;

// The matrix-core path description of the last call, formatted into g_path
// only when it is asked for (gemm_last_path(), GEMM_LOG=debug): tiny GEMMs
// are launch-bound, and formatting it on every call cost about as much host
// time as the rest of the checks.
struct MfmaPath {
  const MfmaTileInfo* ti;
  const char* ops;
  const char* epi;
  bool pingpong, masked, k16_tail, ring;
  int ring_mode;
  int mfold;          // rows folded into the last tile row (ring kernel)
  int atom;           // 16: the two-group kernel on 16x16x32 atoms; 0: the tile's own
  const char* src32;  // "", " f32->f16" or " f32->bf16"
  std::string elem_reason;  // operands read in narrow pieces (general kernel)
  std::string staged;       // operands staged through registers (ring kernel)
};
thread_local MfmaPath g_mpath;
thread_local bool g_path_lazy = false;

const std::string& current_path() {
  if (g_path_lazy) {
    const MfmaPath& m = g_mpath;
    char buf[512], ksplit[32] = "", fold[48] = "";
    if (m.ti->kg > 1) std::snprintf(ksplit, sizeof ksplit, " ksplit%d", m.ti->kg);
    if (m.ring && m.mfold > 0)
      std::snprintf(fold, sizeof fold, " fold(%d row%s)", m.mfold, m.mfold > 1 ? "s" : "");
    const bool a16 = m.atom == 16;
    std::snprintf(buf, sizeof buf, "mfma %s w%dx%d a%dx%dx%d %s epi=%s%s%s%s%s%s%s%s%s%s%s%s%s%s",
                  m.ti->name, m.ti->waves_m,
                  m.pingpong || (m.ring && (m.ring_mode == RING_PP || m.ring_mode == RING_PP_DEEP))
                      ? 4
                      : m.ti->waves_n,
                  a16 ? 16 : m.ti->atom_m, a16 ? 16 : m.ti->atom_n, a16 ? 32 : m.ti->atom_k,
                  m.ops, m.epi, ksplit,
                  m.pingpong ? " pingpong" : "",
                  !m.ring ? ""
                  : m.ring_mode == RING_KSPLIT2 ? " ring ksplit2"
                  : m.ring_mode == RING_DEEP ? " ring deep"
                  : m.ring_mode == RING_PP ? " ring two-group"
                  : m.ring_mode == RING_PP_DEEP ? " ring two-group deep" : " ring",
                  fold, m.masked ? " masked" : "", m.k16_tail ? " k16-tail" : "", m.src32,
                  m.elem_reason.empty() ? "" : " narrow staging (", m.elem_reason.c_str(),
                  m.elem_reason.empty() ? "" : ")",
                  m.staged.empty() ? "" : " staged (", m.staged.c_str(),
                  m.staged.empty() ? "" : ")");
    g_path = buf;
    g_path_lazy = false;
  }
  return g_path;
}

// The library's environment switches, read in one pass over the environment
// at the start of each call (three getenv scans cost more than the checks).
struct EnvSwitches {
  const char* force_path = nullptr;  // GEMM_FORCE_PATH
  const char* force_tile = nullptr;  // GEMM_FORCE_TILE
  const char* log = nullptr;         // GEMM_LOG
  const char* ring_mode = nullptr;   // GEMM_RING_MODE: form of the 128x128 ring kernel
  const char* stage_depth = nullptr; // GEMM_STAGE_DEPTH: slices of staged loads ahead (1 or 2)
};
thread_local EnvSwitches g_env;

void read_env() {
  g_env = EnvSwitches{};
  for (char** e = environ; e && *e; ++e) {
    const char* v = *e;
    if (v[0] != 'G' || std::strncmp(v, "GEMM_", 5) != 0) continue;
    v += 5;
    if (std::strncmp(v, "FORCE_PATH=", 11) == 0) g_env.force_path = v + 11;
    else if (std::strncmp(v, "FORCE_TILE=", 11) == 0) g_env.force_tile = v + 11;
    else if (std::strncmp(v, "LOG=", 4) == 0) g_env.log = v + 4;
    else if (std::strncmp(v, "RING_MODE=", 10) == 0) g_env.ring_mode = v + 10;
    else if (std::strncmp(v, "STAGE_DEPTH=", 12) == 0) g_env.stage_depth = v + 12;
  }
  if (g_env.force_path && !*g_env.force_path) g_env.force_path = nullptr;
  if (g_env.force_tile && !*g_env.force_tile) g_env.force_tile = nullptr;
  if (g_env.log && !*g_env.log) g_env.log = nullptr;
  if (g_env.ring_mode && !*g_env.ring_mode) g_env.ring_mode = nullptr;
  if (g_env.stage_depth && !*g_env.stage_depth) g_env.stage_depth = nullptr;
}

// Largest dimension the int32 index arithmetic in the kernels supports.
constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1024;

struct Plan {
  bool noop = false;        // M == 0 or N == 0
  bool scale_only = false;  // K == 0 or alpha == 0: D = beta*C
  bool mfma = false;
  int tile = 0;
  bool masked = false;
  bool pp_f32 = false;  // float32 operands on the two-group kernel
  bool ring = false;    // 16-bit operands on the 128x128 direct-to-LDS ring kernel
  int epi = EPI_BETA0;
  GemmArgs args{};
  bool byte8 = false;  // 8-bit float operands: the 1-byte-operand kernel
  int byte_kind = 0;
  GemmByteArgs bargs{};
};

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

// Byte extent of a row-major [rows, cols] matrix with leading dimension ld.
unsigned __int128 extent_bytes(int64_t rows, int64_t cols, int64_t ld, int elem) {
  if (rows <= 0 || cols <= 0) return 0;
  return ((unsigned __int128)(rows - 1) * (unsigned __int128)ld + (unsigned __int128)cols) *
         (unsigned __int128)elem;
}

bool overlaps(const void* p, unsigned __int128 np, const void* q, unsigned __int128 nq) {
  if (np == 0 || nq == 0) return false;
  const unsigned __int128 a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + nq && b < a + np;
}

// Widest staging load (in elements of esz bytes, at most 16 bytes) whose byte
// size divides both the operand's base address and its row pitch.
int vector_width(const void* ptr, int64_t ld, int esz) {
  int vw = 16 / esz;
  while (vw > 1 && ((uintptr_t)ptr % (esz * vw) != 0 || (ld * esz) % (esz * vw) != 0)) vw /= 2;
  return vw;
}

std::string pitch_reason(const char* name, const void* ptr, int64_t ld, int vw, int esz) {
  char buf[160];
  if ((uintptr_t)ptr % 16 != 0) {
    std::snprintf(buf, sizeof buf, "%s: %d-byte loads, base address is not 16-byte aligned",
                  name, esz * vw);
  } else {
    std::snprintf(buf, sizeof buf, "%s: %d-byte loads, row pitch %lld B is not a multiple of 16 B",
                  name, esz * vw, (long long)(ld * esz));
  }
  return buf;
}

// Largest tile that still gives every CU work; grids that even 64x64 tiles
// leave under-filled (fewer than 256 tiles) take 32x32 tiles with K split
// over four wave groups once K holds a step of 64 for each group.
// Tiles per round of the 256x256 grid (one workgroup per CU).
constexpr int64_t kPpEdgeRound = 256;

// whole64k4: the 64x64 four-group tile may be chosen (it runs whole tiles only).
int choose_tile(int64_t M, int64_t N, int64_t K, bool whole64k4 = true) {
  auto count = [&](int t) {
    const MfmaTileInfo& ti = mfma_tile_info(t);
    return ((M + ti.bm - 1) / ti.bm) * ((N + ti.bn - 1) / ti.bn);
  };
  // 256x256 tiles also on grids that leave CUs idle, once K is long enough
  // for their twice larger work per loaded byte to outweigh the idle CUs
  // (measured against the 128x128 two-group form, same box, bf16: 192
  // tiles 1.41x faster at K = 2048, 1.53-1.61x at K = 4096-8192; 128 tiles
  // 1.03-1.11x at K = 2048-8192, 0.96x at K = 1024).
  const int64_t n256 = count(TILE_256x256);
  if (n256 >= 256 || (n256 >= 192 && K >= 1024) || (n256 >= 128 && K >= 2048))
    return TILE_256x256;
  if (count(TILE_128x128) >= 128) return TILE_128x128;
  if (M <= 16 && N <= 16) return TILE_16x16;
  const MfmaTileInfo& k4 = mfma_tile_info(TILE_32x32K4);
  // K split over one-wave groups when 64x64 tiles would leave CUs idle, or
  // fill exactly one round with a K long enough that each 64x64 tile's chain
  // of dependent slices dominates (measured, same box, 256 tiles of 64x64:
  // 1024^2 x 4096 NT 34.8 -> 27.9 us, 128x8192x8192 NT 64 -> 49 us, 96 x
  // 8192 x 8192 99 -> 48 us; at K = 1024-2048 the 64x64 tile was as fast or
  // faster).
  const int64_t n64 = count(TILE_64x64);
  // One round of 64x64 tiles (192-256) with K >= 2048: those tiles with K
  // split over four groups of 2x2 waves, when the call needs no masking
  // (measured, same box: 128x8192x8192 NT 49.0 -> 36.6 us against 32x32
  // tiles in four K groups, NN 63.2 -> 40.5; 1024^2 x 4096 27.9 -> 21.2;
  // 1024^2 x 2048 16.4 -> 13.1 against 64x64 tiles; with 128 tiles of 64x64
  // the 32x32 tiles stay faster: 64x8192x8192 28.7 against 36.4 us).
  if (whole64k4 && n64 >= 192 && n64 <= 256 && K >= 2048) return TILE_64x64K4;
  if ((n64 < 256 || (n64 == 256 && K >= 4096)) && K >= (int64_t)k4.bk * k4.kg) {
    // Eight K groups when the 32x32 tiles fit one round (the eight-group
    // workgroup takes 128 KiB of LDS, so one per CU) and each group still
    // walks at least four slices: the shorter chain of dependent slice loads
    // per wave measured 1x4097x4096 15.1 -> 11.6 us, 4096x1x4096 18.4 ->
    // 12.2, 256x1024x4096 10.8 -> 9.7; past one round (1x8193x8192: 257
    // tiles) four groups stay faster (28.4 against 39.2 us).
    if (count(TILE_32x32K8) <= 256 && K >= 2048) return TILE_32x32K8;
    return TILE_32x32K4;
  }
  return TILE_64x64;
}

// Whole 256x256 tiles of a 1-byte-operand call, in any layout, take the
// two-group kernel (K a multiple of its 128-byte slices, 16-byte operand and
// C/D rows, 32-bit load offsets).
bool byte_pingpong(const GemmByteArgs& b) {
  const int t = byte_pp_tile();
  const int64_t ldmax = b.lda > b.ldb ? b.lda : b.ldb;
  return b.M % t == 0 && b.N % t == 0 && b.K > 0 && b.K % 128 == 0 && b.a_vec16 && b.b_vec16 &&
         b.cd_vec16 && ldmax * t + 4096 < (int64_t{1} << 31);
}

// Other 1-byte-operand calls also take the two-group kernel, with edge tiles
// (pieces outside the operands read as zeros, C and D accessed inside
// M x N only), when K is a multiple of 16, an M/N-contiguous operand's
// contiguous dimension of 16 (whole 16-byte pieces), operand rows are
// 16-byte aligned, and the grid has at least kBytePpMaskedMinTiles tiles of
// 256x256 (smaller grids keep the 128x128 kernel, which spreads them over
// more CUs). C and D go by column quads when their rows are 16-byte aligned
// and N is a multiple of 4, else element by element. Measured against the
// 128x128 kernel, same box: fp8 4000^2 x 4096 NT 111 -> 56 us, TN 181 ->
// 58 us, int8 106 -> 59 us, 8000^2 x 8192 740 -> 379 us, 1008^2 x 1024 NN
// 24.5 -> 19.2 us; 512^3 (4 tiles) equal.
constexpr int64_t kBytePpMaskedMinTiles = 4;
bool byte_pingpong_masked(const GemmByteArgs& b, int transA, int transB) {
  const int64_t t = byte_pp_tile();
  const int64_t ldmax = b.lda > b.ldb ? b.lda : b.ldb;
  const int64_t tiles = ((b.M + t - 1) / t) * ((b.N + t - 1) / t);
  return b.K > 0 && b.K % 16 == 0 && (!transA || b.M % 16 == 0) &&
         (transB || b.N % 16 == 0) && b.a_vec16 && b.b_vec16 &&
         ldmax * t + 4096 < (int64_t{1} << 31) && tiles >= kBytePpMaskedMinTiles;
}

void set_byte_tiles(GemmByteArgs& b, int transA, int transB) {
  b.pingpong = byte_pingpong(b) ? 1 : byte_pingpong_masked(b, transA, transB) ? 2 : 0;
  b.cd_scalar = b.pingpong == 2 && !(b.cd_vec16 && b.N % 4 == 0);
  const int tm = b.pingpong ? byte_pp_tile() : byte_tile_m();
  const int tn = b.pingpong ? byte_pp_tile() : byte_tile_n();
  b.tiles_m = (int)((b.M + tm - 1) / tm);
  b.tiles_n = (int)((b.N + tn - 1) / tn);
}

int plan_call(int64_t M, int64_t N, int64_t K, int dtype, int transA, int transB, float alpha,
              float beta, const void* A, int64_t lda, const void* B, int64_t ldb, const float* C,
              int64_t ldc, const float* D, int64_t ldd, Plan& plan) {
  g_err.clear();
  g_path.clear();
  g_path_lazy = false;
  read_env();
  char buf[256];
  transA = transA != 0;
  transB = transB != 0;
  if (M < 0 || N < 0 || K < 0) {
    std::snprintf(buf, sizeof buf, "negative dimension: M=%lld N=%lld K=%lld", (long long)M,
                  (long long)N, (long long)K);
    return fail(GEMM_ERR_INVALID_ARG, buf);
  }
  if (dtype < GEMM_DTYPE_F16 || dtype > GEMM_DTYPE_F8_E5M2) {
    std::snprintf(buf, sizeof buf,
                  "dtype code %d is none of f16 (0), bf16 (1), f32->f16 (2), f32->bf16 (3), "
                  "fp8 e4m3 (4), fp8 e5m2 (5)", dtype);
    return fail(GEMM_ERR_UNSUPPORTED, buf);
  }
  // f32 operands are rounded to the 16-bit type as they are staged; 8-bit
  // float operands run on the 1-byte-operand kernel.
  const bool fp8 = dtype >= GEMM_DTYPE_F8_E4M3;
  const bool src32 = !fp8 && dtype >= GEMM_DTYPE_F32_F16;
  const int esz = fp8 ? 1 : src32 ? 4 : 2;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) {
    return fail(GEMM_ERR_UNSUPPORTED, "a dimension exceeds 2^31-1024");
  }
  const int64_t min_lda = transA ? M : K, min_ldb = transB ? K : N;
  if (lda < (min_lda > 1 ? min_lda : 1)) {
    std::snprintf(buf, sizeof buf, "lda=%lld is smaller than %s=%lld", (long long)lda,
                  transA ? "M" : "K", (long long)min_lda);
    return fail(GEMM_ERR_INVALID_ARG, buf);
  }
  if (ldb < (min_ldb > 1 ? min_ldb : 1)) {
    std::snprintf(buf, sizeof buf, "ldb=%lld is smaller than %s=%lld", (long long)ldb,
                  transB ? "K" : "N", (long long)min_ldb);
    return fail(GEMM_ERR_INVALID_ARG, buf);
  }
  if (ldd < (N > 1 ? N : 1)) {
    std::snprintf(buf, sizeof buf, "ldd=%lld is smaller than N=%lld", (long long)ldd,
                  (long long)N);
    return fail(GEMM_ERR_INVALID_ARG, buf);
  }
  const bool reads_c = beta != 0.0f;
  if (reads_c && ldc < (N > 1 ? N : 1)) {
    std::snprintf(buf, sizeof buf, "ldc=%lld is smaller than N=%lld", (long long)ldc,
                  (long long)N);
    return fail(GEMM_ERR_INVALID_ARG, buf);
  }
  if (M == 0 || N == 0) {
    plan.noop = true;
    g_path = "noop: empty output";
    return GEMM_OK;
  }
  const bool reads_ab = K > 0 && alpha != 0.0f;
  if (!D) return fail(GEMM_ERR_INVALID_ARG, "D is NULL");
  if ((uintptr_t)D % 4) return fail(GEMM_ERR_INVALID_ARG, "D is not 4-byte aligned");
  if (reads_c && !C) return fail(GEMM_ERR_INVALID_ARG, "C is NULL but beta != 0");
  if (reads_c && (uintptr_t)C % 4) return fail(GEMM_ERR_INVALID_ARG, "C is not 4-byte aligned");
  if (reads_ab && (!A || !B)) return fail(GEMM_ERR_INVALID_ARG, "A or B is NULL");
  if (reads_ab && ((uintptr_t)A % esz || (uintptr_t)B % esz))
    return fail(GEMM_ERR_INVALID_ARG, src32 ? "A or B is not 4-byte aligned" : "A or B is not 2-byte aligned");

  // Aliasing: D is written, so it must not overlap anything it is computed
  // from, except C itself in the exact in-place form.
  const unsigned __int128 d_ext = extent_bytes(M, N, ldd, 4);
  if (reads_c) {
    const unsigned __int128 c_ext = extent_bytes(M, N, ldc, 4);
    const bool same = (const void*)C == (const void*)D && ldc == ldd;
    if (!same && overlaps(C, c_ext, D, d_ext))
      return fail(GEMM_ERR_ALIAS, "D overlaps C without being the same matrix (C == D and "
                                  "ldc == ldd is the only allowed overlap)");
  }
  if (reads_ab) {
    const unsigned __int128 a_ext =
        extent_bytes(transA ? K : M, transA ? M : K, lda, esz);
    const unsigned __int128 b_ext =
        extent_bytes(transB ? N : K, transB ? K : N, ldb, esz);
    if (overlaps(A, a_ext, D, d_ext)) return fail(GEMM_ERR_ALIAS, "D overlaps A");
    if (overlaps(B, b_ext, D, d_ext)) return fail(GEMM_ERR_ALIAS, "D overlaps B");
  }

  GemmArgs& a = plan.args;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = const_cast<float*>(D);
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = reads_c ? ldc : ldd;
  a.ldd = ldd;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.alpha = alpha;
  a.beta = beta;
  a.group_m = 8;
  a.wide_epi = ((uintptr_t)D % 16 == 0 && ldd % 4 == 0 &&
                (!reads_c || ((uintptr_t)C % 16 == 0 && ldc % 4 == 0)))
                   ? 1
                   : 0;
  plan.epi = !reads_c ? EPI_BETA0 : (alpha == 1.0f && beta == 1.0f ? EPI_ACC_PLUS_C : EPI_GENERAL);
  a.epi = plan.epi;
  const char* epi_name = plan.epi == EPI_BETA0 ? "beta0" : plan.epi == EPI_ACC_PLUS_C ? "acc+c" : "general";

  if (!reads_ab) {
    plan.scale_only = true;
    std::snprintf(buf, sizeof buf, "scale: D = beta*C (%s)", K == 0 ? "K == 0" : "alpha == 0");
    g_path = buf;
    return GEMM_OK;
  }

  if (fp8) {
    if (const char* force = g_env.force_path) {
      if (std::strcmp(force, "fma") == 0)
        return fail(GEMM_ERR_UNSUPPORTED, "GEMM_FORCE_PATH=fma has no 8-bit float form");
      if (std::strcmp(force, "mfma") != 0)
        return fail(GEMM_ERR_INVALID_ARG,
                    std::string("GEMM_FORCE_PATH must be mfma or fma, got ") + force);
    }
    GemmByteArgs& b = plan.bargs;
    b.A = A;
    b.B = B;
    b.C = C;
    b.D = const_cast<float*>(D);
    b.lda = lda;
    b.ldb = ldb;
    b.ldc = a.ldc;
    b.ldd = ldd;
    b.M = (int)M;
    b.N = (int)N;
    b.K = (int)K;
    b.alpha_f = alpha;
    b.beta_f = beta;
    b.read_c = reads_c ? 1 : 0;
    b.a_vec16 = ((uintptr_t)A % 16 == 0 && lda % 16 == 0) ? 1 : 0;
    b.b_vec16 = ((uintptr_t)B % 16 == 0 && ldb % 16 == 0) ? 1 : 0;
    b.cd_vec16 = ((uintptr_t)D % 16 == 0 && ldd % 4 == 0 &&
                  (!reads_c || ((uintptr_t)C % 16 == 0 && a.ldc % 4 == 0))) ? 1 : 0;
    set_byte_tiles(b, transA, transB);
    b.group_m = 8;
    if ((int64_t)b.tiles_m * b.tiles_n > 0x7fffffff)
      return fail(GEMM_ERR_UNSUPPORTED, "too many output tiles for one launch");
    plan.byte8 = true;
    plan.byte_kind = dtype == GEMM_DTYPE_F8_E4M3 ? BYTE_F8E4M3 : BYTE_F8E5M2;
    const char* ops8 = transA ? (transB ? "TT" : "TN") : (transB ? "NT" : "NN");
    const int t8 = b.pingpong ? byte_pp_tile() : byte_tile_m();
    std::snprintf(buf, sizeof buf, "fp8 %s mfma t%dx%dx128 %s %s %s epi=%s%s%s%s",
                  dtype == GEMM_DTYPE_F8_E4M3 ? "e4m3" : "e5m2", t8, t8,
                  b.pingpong ? "w2x4" : "w2x2", b.pingpong ? "a16x16x128" : "a32x32x64", ops8,
                  epi_name, b.pingpong == 2 ? " pingpong masked" : b.pingpong ? " pingpong" : "",
                  b.cd_scalar ? " elementwise C/D" : "",
                  (!b.a_vec16 || !b.b_vec16) ? " bytewise staging" : "");
    g_path = buf;
    return GEMM_OK;
  }

  // Path selection. The matrix-core path stages A and B in 16-byte pieces; an
  // operand whose base or row pitch is not a multiple of 16 bytes is read with
  // the widest loads they allow (8, 4 or 2 bytes, masked kernel), so every
  // f16/bf16 call runs on the matrix cores unless the VALU path is forced.
  const int a_vw = vector_width(A, lda, esz), b_vw = vector_width(B, ldb, esz);
  const bool a_elem = a_vw * esz < 16, b_elem = b_vw * esz < 16;
  std::string elem_reason;
  if (a_elem) elem_reason = pitch_reason("A", A, lda, a_vw, esz);
  if (b_elem) elem_reason += (a_elem ? "; " : "") + pitch_reason("B", B, ldb, b_vw, esz);
  std::string decline;
  const char* force = g_env.force_path;
  if (force && std::strcmp(force, "fma") == 0) {
    if (src32)
      return fail(GEMM_ERR_UNSUPPORTED, "GEMM_FORCE_PATH=fma has no f32-operand form");
    decline = "forced by GEMM_FORCE_PATH=fma";
  } else if (force && std::strcmp(force, "mfma") != 0) {
    return fail(GEMM_ERR_INVALID_ARG, std::string("GEMM_FORCE_PATH must be mfma or fma, got ") + force);
  }
  const char* ops = transA ? (transB ? "TT" : "TN") : (transB ? "NT" : "NN");

  if (!decline.empty()) {
    plan.mfma = false;
    a.tiles_m = (int)((M + kFmaTileM - 1) / kFmaTileM);
    a.tiles_n = (int)((N + kFmaTileN - 1) / kFmaTileN);
    std::snprintf(buf, sizeof buf, "fma t%dx%dx16 %s epi=%s: %s", kFmaTileM, kFmaTileN, ops,
                  epi_name, decline.c_str());
    g_path = buf;
    return GEMM_OK;
  }

  int tile = choose_tile(M, N, K);
  if (const char* ft = g_env.force_tile) {
    int found = -1;
    for (int t = 0; t < NUM_MFMA_TILES; ++t)
      if (std::strcmp(ft, mfma_tile_info(t).name) == 0) found = t;
    if (found < 0)
      return fail(GEMM_ERR_INVALID_ARG, std::string("GEMM_FORCE_TILE names no tile: ") + ft);
    tile = found;
  }
  a.a_vw = a_vw;
  a.b_vw = b_vw;
  a.src32 = src32 ? (dtype == GEMM_DTYPE_F32_BF16 ? 2 : 1) : 0;
  // Whether tile t needs the masked kernel (edges, a K tail, narrow staging,
  // float32 operands off the two-group kernel) and whether its operand boxes
  // need 64-bit addressing: the unmasked kernels address a box through a
  // buffer resource with 32-bit byte offsets spanning up to max(bm, bn, bk)
  // rows of the operand; larger pitches take the masked kernel's 64-bit
  // addressing. With K groups, the unmasked kernel needs every group's every
  // step whole.
  bool big_pitch = false;
  auto plan_tile = [&](int t) {
    const MfmaTileInfo& ti = mfma_tile_info(t);
    plan.masked = (M % ti.bm) || (N % ti.bn) || (K % ((int64_t)ti.bk * ti.kg));
    const int64_t rows = ti.bm > ti.bn ? (ti.bm > ti.bk ? ti.bm : ti.bk)
                                       : (ti.bn > ti.bk ? ti.bn : ti.bk);
    const int64_t ldmax = lda > ldb ? lda : ldb;
    big_pitch = ldmax * esz * rows + 4096 >= (int64_t{1} << 31);
    if (big_pitch) plan.masked = true;
    // Float32 operands with 16-byte rows, whole 256x256 tiles and K a
    // multiple of its 32-deep slices, any layout: the two-group kernel rounds
    // them as it reads fragments (edge tiles: see below). Every other float32
    // call is rounded while it is staged (ring kernel, or the masked kernel
    // for 64-bit pitches).
    plan.pp_f32 = src32 && t == TILE_256x256 && !a_elem && !b_elem &&
                  !big_pitch && M % ti.bm == 0 && N % ti.bn == 0 && K % pp_f32_slice() == 0;
    if (plan.pp_f32) plan.masked = false;
    else if (a_elem || b_elem || src32) plan.masked = true;
  };
  plan_tile(tile);
  // The 256x256 tile runs on the two-group kernel: whole tiles, or edge
  // tiles whose operands load in whole 16-byte pieces (16-byte rows, each
  // operand's contiguous dimension a multiple of 8 16-bit or 4 float32
  // values, 32-bit offsets) when the grid fills its last round of 256 CUs to
  // at least 3/4 (forced 256x256 tiles skip that test); other calls that
  // need masking at that size take the 128x128 kernels.
  // The 64x64 four-group tile runs whole tiles only; a call that needs
  // masking takes the tile chosen without it.
  if (tile == TILE_64x64K4 && plan.masked) {
    tile = choose_tile(M, N, K, false);
    plan_tile(tile);
  }
  if (tile == TILE_256x256 && plan.masked) {
    const MfmaTileInfo& t256 = mfma_tile_info(TILE_256x256);
    const int64_t n256 = ((M + t256.bm - 1) / t256.bm) * ((N + t256.bn - 1) / t256.bn);
    const int64_t rounds = (n256 + kPpEdgeRound - 1) / kPpEdgeRound;
    const bool fills = g_env.force_tile || 4 * n256 >= 3 * rounds * kPpEdgeRound;
    const int64_t q = 16 / esz;  // elements per 16-byte piece
    const bool edges = !a_elem && !b_elem && !big_pitch &&
                       (transA ? M % q == 0 : K % q == 0) && (transB ? K % q == 0 : N % q == 0);
    if (edges && fills) {
      plan.pp_f32 = src32;  // float32 operands: the f32 form of the kernel, masked
    } else {
      tile = TILE_128x128;
      plan_tile(tile);
    }
  }
  const MfmaTileInfo& ti = mfma_tile_info(tile);
  plan.mfma = true;
  plan.tile = tile;
  a.a_fast = !src32 && !big_pitch;
  a.b_fast = !src32 && !big_pitch;
  a.tiles_m = (int)((M + ti.bm - 1) / ti.bm);
  a.tiles_n = (int)((N + ti.bn - 1) / ti.bn);
  if ((int64_t)a.tiles_m * a.tiles_n > 0x7fffffff)
    return fail(GEMM_ERR_UNSUPPORTED, "too many output tiles for one launch");
  // 256x256 tiles (any operand layout) take the kernel with two wave groups
  // (2x4 waves) and direct global->LDS loads.
  const bool pingpong = tile == TILE_256x256;  // includes plan.pp_f32
  // 128x128 tiles of 16-bit operands take the direct-to-LDS ring kernel,
  // edges, K tails and unaligned rows included; each operand is loaded
  // straight into LDS when its base and row pitch are multiples of 16 bytes
  // and the edges cutting its contiguous dimension fall on multiples of 8
  // elements, else staged through registers.
  std::string staged;
  // Float32 operands off the two-group kernel's NT fast path take the ring
  // kernel too, both staged through registers and rounded there.
  plan.ring = tile == TILE_128x128 && !big_pitch;
  if (plan.ring) {
    auto direct = [&](int vw, bool mn_contig, int64_t mn) {
      return vw == 8 && (mn_contig ? mn % 8 == 0 : K % 8 == 0);
    };
    a.a_direct = !src32 && direct(a_vw, transA != 0, M) ? 1 : 0;
    a.b_direct = !src32 && direct(b_vw, transB == 0, N) ? 1 : 0;
    auto why = [&](const char* name, const void* ptr, int64_t ld, int vw, bool mn_contig) {
      char w[160];
      if (vw != 8) {
        if ((uintptr_t)ptr % 16 != 0)
          std::snprintf(w, sizeof w, "%s: base address is not 16-byte aligned", name);
        else
          std::snprintf(w, sizeof w, "%s: row pitch %lld B is not a multiple of 16 B", name,
                        (long long)(ld * 2));
      } else {
        std::snprintf(w, sizeof w, "%s: %s %% 8 != 0", name,
                      mn_contig ? (name[0] == 'A' ? "M" : "N") : "K");
      }
      return std::string(w);
    };
    if (src32) {
      staged = "A, B: float32 values rounded in registers";
    } else {
      if (!a.a_direct) staged = why("A", A, lda, a_vw, transA != 0);
      if (!a.b_direct) staged += (staged.empty() ? "" : "; ") + why("B", B, ldb, b_vw, transB == 0);
    }
    elem_reason.clear();
    // "masked": edge tiles or a K tail (the ring kernel masks in place)
    plan.masked = (M % ti.bm) || (N % ti.bn) || (K % ti.bk);
    // Both operands straight into LDS: two wave groups taking turns (five
    // half-slots, two workgroups per CU) on grids of more than one tile per
    // CU; on smaller grids the deep ring (one wave per SIMD, every slice
    // requested four ahead from 160 KiB), except with B N-contiguous and a
    // long K, where the two-group form with ten half-slots hides the
    // transposed B reads behind the second wave per SIMD (measured, NN and
    // TN: 8-15 % faster at K = 2048, 5-8 % slower at K = 1024, where the
    // deep ring's earlier start counts more; slower with B K-contiguous). A
    // staged operand: K split over two wave groups per workgroup (8 waves,
    // two rings) on small grids, so that each SIMD still alternates between
    // two waves; one group per workgroup and two workgroups per CU beyond.
    int64_t ntiles = (int64_t)a.tiles_m * a.tiles_n;
    const bool both_direct = a.a_direct && a.b_direct;
    // A staged operand and up to 4 rows past the last whole tile row that
    // alone push the grid past one tile per CU: the last tile row computes
    // them (one more row of 16x16x32 atoms, A read element by element), so
    // the grid keeps one tile per CU and takes the two-K-group form.
    a.mfold = 0;
    const int64_t mrem = M % ti.bm;
    if (!src32 && !both_direct && mrem >= 1 && mrem <= 4 && M >= ti.bm) {
      const int64_t folded = (M / ti.bm) * a.tiles_n;
      if (ntiles > 256 && folded <= 256) {
        a.mfold = (int)mrem;
        a.tiles_m = (int)(M / ti.bm);
        ntiles = folded;
      }
    }
    a.ring_mode = ntiles > 256 ? (both_direct ? RING_PP : RING_SHARED)
                  : !both_direct ? RING_KSPLIT2
                  : (transB || K < 2048) ? RING_DEEP : RING_PP_DEEP;
    if (const char* rm = g_env.ring_mode) {
      if (std::strcmp(rm, "shared") == 0) a.ring_mode = RING_SHARED;
      else if (std::strcmp(rm, "ksplit2") == 0) a.ring_mode = RING_KSPLIT2;
      else if (std::strcmp(rm, "deep") == 0 && a.a_direct && a.b_direct) a.ring_mode = RING_DEEP;
      else if (std::strcmp(rm, "pp") == 0 && a.a_direct && a.b_direct) a.ring_mode = RING_PP;
      else if (std::strcmp(rm, "ppdeep") == 0 && a.a_direct && a.b_direct)
        a.ring_mode = RING_PP_DEEP;
      else if (std::strcmp(rm, "deep") == 0 || std::strcmp(rm, "pp") == 0 ||
               std::strcmp(rm, "ppdeep") == 0)
        return fail(GEMM_ERR_UNSUPPORTED, std::string("GEMM_RING_MODE=") + rm +
                                              " needs both operands loaded straight into LDS");
      else
        return fail(GEMM_ERR_INVALID_ARG,
                    std::string("GEMM_RING_MODE must be shared, ksplit2, deep, pp or ppdeep, got ") +
                        rm);
    }
    if (a.mfold > 0 && a.ring_mode != RING_KSPLIT2) {  // a forced form: no folded rows
      a.mfold = 0;
      a.tiles_m = (int)((M + ti.bm - 1) / ti.bm);
    }
    // One staged 16-bit operand (shared ring or two K groups): its loads go
    // three slices ahead into two register sets (GEMM_STAGE_DEPTH=1: two
    // slices ahead, one set).
    a.stage_depth = 2;
    if (const char* sd = g_env.stage_depth) {
      if (std::strcmp(sd, "1") == 0) a.stage_depth = 1;
      else if (std::strcmp(sd, "2") != 0)
        return fail(GEMM_ERR_INVALID_ARG, std::string("GEMM_STAGE_DEPTH must be 1 or 2, got ") + sd);
    }
  }
  // A last K step whose valid part ends within the first half of a 16x16x32
  // sub-step finishes with v_mfma_f32_16x16x16 (no product of staged zeros).
  const bool k16_tail = ti.atom_k == 32 && K % 32 >= 1 && K % 32 <= 16;
  g_mpath.ti = &ti;
  g_mpath.ops = ops;
  g_mpath.epi = epi_name;
  g_mpath.pingpong = pingpong;
  // The two-group kernel for 16-bit operands multiplies on 16x16x32 atoms
  // when A is K-contiguous (see gemm_mfma_pingpong.h).
  g_mpath.atom = pingpong && !plan.pp_f32 && !transA ? 16 : 0;
  g_mpath.ring = plan.ring;
  g_mpath.ring_mode = a.ring_mode;
  g_mpath.mfold = plan.ring ? a.mfold : 0;
  g_mpath.staged.swap(staged);
  g_mpath.masked = plan.masked;
  g_mpath.k16_tail = k16_tail;
  g_mpath.src32 = !src32 ? "" : dtype == GEMM_DTYPE_F32_BF16 ? " f32->bf16" : " f32->f16";
  g_mpath.elem_reason.swap(elem_reason);
  g_path_lazy = true;
  return GEMM_OK;
}

// Checks and launch arguments of the int8 form (same rules as the float form,
// with 1-byte operands and int32 C/D).
int plan_i8(int64_t M, int64_t N, int64_t K, int transA, int transB, int32_t alpha, int32_t beta,
            const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const int32_t* C,
            int64_t ldc, const int32_t* D, int64_t ldd, GemmByteArgs& a, bool& noop) {
  g_err.clear();
  g_path.clear();
  g_path_lazy = false;
  read_env();
  noop = false;
  char buf[256];
  transA = transA != 0;
  transB = transB != 0;
  if (M < 0 || N < 0 || K < 0) {
    std::snprintf(buf, sizeof buf, "negative dimension: M=%lld N=%lld K=%lld", (long long)M,
                  (long long)N, (long long)K);
    return fail(GEMM_ERR_INVALID_ARG, buf);
  }
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(GEMM_ERR_UNSUPPORTED, "a dimension exceeds 2^31-1024");
  const int64_t min_lda = transA ? M : K, min_ldb = transB ? K : N;
  if (lda < (min_lda > 1 ? min_lda : 1) || ldb < (min_ldb > 1 ? min_ldb : 1) ||
      ldd < (N > 1 ? N : 1))
    return fail(GEMM_ERR_INVALID_ARG, "a leading dimension is smaller than its row length");
  const bool reads_c = beta != 0;
  if (reads_c && ldc < (N > 1 ? N : 1))
    return fail(GEMM_ERR_INVALID_ARG, "ldc is smaller than N");
  if (M == 0 || N == 0) {
    noop = true;
    g_path = "noop: empty output";
    return GEMM_OK;
  }
  const bool reads_ab = K > 0 && alpha != 0;
  if (!D) return fail(GEMM_ERR_INVALID_ARG, "D is NULL");
  if ((uintptr_t)D % 4) return fail(GEMM_ERR_INVALID_ARG, "D is not 4-byte aligned");
  if (reads_c && !C) return fail(GEMM_ERR_INVALID_ARG, "C is NULL but beta != 0");
  if (reads_c && (uintptr_t)C % 4) return fail(GEMM_ERR_INVALID_ARG, "C is not 4-byte aligned");
  if (reads_ab && (!A || !B)) return fail(GEMM_ERR_INVALID_ARG, "A or B is NULL");
  const unsigned __int128 d_ext = extent_bytes(M, N, ldd, 4);
  if (reads_c) {
    const bool same = (const void*)C == (const void*)D && ldc == ldd;
    if (!same && overlaps(C, extent_bytes(M, N, ldc, 4), D, d_ext))
      return fail(GEMM_ERR_ALIAS, "D overlaps C without being the same matrix (C == D and "
                                  "ldc == ldd is the only allowed overlap)");
  }
  if (reads_ab) {
    if (overlaps(A, extent_bytes(transA ? K : M, transA ? M : K, lda, 1), D, d_ext))
      return fail(GEMM_ERR_ALIAS, "D overlaps A");
    if (overlaps(B, extent_bytes(transB ? N : K, transB ? K : N, ldb, 1), D, d_ext))
      return fail(GEMM_ERR_ALIAS, "D overlaps B");
  }
  a = GemmByteArgs{};
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = const_cast<int32_t*>(D);
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = reads_c ? ldc : ldd;
  a.ldd = ldd;
  a.M = (int)M;
  a.N = (int)N;
  a.K = reads_ab ? (int)K : 0;  // no K loop when the product does not contribute
  a.alpha_i = alpha;
  a.beta_i = beta;
  a.read_c = reads_c ? 1 : 0;
  a.a_vec16 = ((uintptr_t)A % 16 == 0 && lda % 16 == 0) ? 1 : 0;
  a.b_vec16 = ((uintptr_t)B % 16 == 0 && ldb % 16 == 0) ? 1 : 0;
  a.cd_vec16 = ((uintptr_t)D % 16 == 0 && ldd % 4 == 0 &&
                (!reads_c || ((uintptr_t)C % 16 == 0 && ldc % 4 == 0))) ? 1 : 0;
  set_byte_tiles(a, transA, transB);
  a.group_m = 8;
  if ((int64_t)a.tiles_m * a.tiles_n > 0x7fffffff)
    return fail(GEMM_ERR_UNSUPPORTED, "too many output tiles for one launch");
  const char* ops = transA ? (transB ? "TT" : "TN") : (transB ? "NT" : "NN");
  const int t8 = a.pingpong ? byte_pp_tile() : byte_tile_m();
  std::snprintf(buf, sizeof buf, "i8 mfma t%dx%dx128 %s %s %s epi=%s%s%s%s%s", t8, t8,
                a.pingpong ? "w2x4" : "w2x2", a.pingpong ? "a16x16x64" : "a32x32x32", ops,
                reads_c ? "general" : "beta0",
                a.pingpong == 2 ? " pingpong masked" : a.pingpong ? " pingpong" : "",
                a.cd_scalar ? " elementwise C/D" : "",
                reads_ab ? "" : " (K == 0 or alpha == 0: D = beta*C)",
                (reads_ab && (!a.a_vec16 || !a.b_vec16)) ? " bytewise staging" : "");
  g_path = buf;
  return GEMM_OK;
}

// Launch a planned call.
hipError_t launch_plan(const Plan& plan, int dtype, int transA, int transB, hipStream_t s) {
  if (plan.noop) return hipSuccess;
  if (plan.scale_only) return launch_scale_c(plan.args, s);
  if (plan.byte8) return launch_byte(plan.byte_kind, transA != 0, transB != 0, plan.bargs, s);
  if (plan.pp_f32)
    return launch_pp_f32(dtype & 1, transA != 0, transB != 0, plan.masked, plan.args, s);
  if (plan.ring) return launch_ring128(dtype & 1, transA != 0, transB != 0, plan.args, s);
  if (plan.mfma)
    return launch_mfma(plan.tile, dtype & 1, transA != 0, transB != 0, plan.masked, plan.args, s);
  return launch_fma(dtype, transA != 0, transB != 0, plan.args, s);
}

// Ragged shapes just past a multiple of the 256x256 tile: when at most
// kSplitMaxRem rows and columns past the last whole tile push a grid of at
// least one round of 256 whole tiles into one more round, the call runs as
// three: the whole tiles (two-group kernel), the remainder rows
// under all columns, and the remainder columns beside the whole rows, each
// planned like a call of its own and launched in that order on the stream.
// Every element of D is computed once, by one of the three. Measured, same
// box, bf16 NT: 4097^2 x 4096 one launch on 128x128 tiles 193 us, the
// pieces 103.5 + 15.0 + 18.5 us; 8193^2 x 8192 masked 256x256 tiles 932 us,
// the pieces 733 + 28.5 + 33.9 us; with 64, 104 and 128 remainder rows and
// columns (K = 4096) one launch takes 198 us against 107 us for the whole
// tiles plus 32, 50 and 43 us for the two strips.
constexpr int64_t kSplitMaxRem = 128;

struct SplitPart {
  const char* what;  // "core", "rows" or "cols"
  int64_t M, N;
  const void* A;
  const void* B;
  const float* C;
  const float* D;
};

// The parts (core, then rows, then columns; empty parts left out) if the
// call is split, else 0 parts. `full` is the plan of the whole call.
int plan_split(int64_t M, int64_t N, int dtype, int transA, int transB, const void* A,
               int64_t lda, const void* B, int64_t ldb, const float* C, int64_t ldc,
               const float* D, int64_t ldd, const Plan& full, SplitPart (&part)[3]) {
  if (g_env.force_path || g_env.force_tile || g_env.ring_mode) return 0;
  if (full.noop || full.scale_only || full.byte8 || !full.mfma) return 0;
  const bool src32 = dtype >= GEMM_DTYPE_F32_F16;
  const int esz = src32 ? 4 : 2;
  const MfmaTileInfo& t = mfma_tile_info(TILE_256x256);
  const int64_t rm = M % t.bm, rn = N % t.bn, Mc = M - rm, Nc = N - rn;
  if ((rm == 0 && rn == 0) || rm > kSplitMaxRem || rn > kSplitMaxRem || Mc == 0 || Nc == 0)
    return 0;
  const int64_t core = (Mc / t.bm) * (Nc / t.bn);
  const int64_t all = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
  if (core < kPpEdgeRound || (core + kPpEdgeRound - 1) / kPpEdgeRound ==
                                 (all + kPpEdgeRound - 1) / kPpEdgeRound)
    return 0;
  // Both operands in whole 16-byte rows, so the core takes the two-group
  // kernel and the parts' pointers keep that alignment.
  if (vector_width(A, lda, esz) * esz < 16 || vector_width(B, ldb, esz) * esz < 16) return 0;
  const char* a = static_cast<const char*>(A);
  const char* b = static_cast<const char*>(B);
  int n = 0;
  part[n++] = SplitPart{"core", Mc, Nc, A, B, C, D};
  if (rm > 0)
    part[n++] = SplitPart{"rows", rm, N, transA ? a + Mc * esz : a + Mc * lda * esz, B,
                          C ? C + Mc * ldc : nullptr, D + Mc * ldd};
  if (rn > 0)
    part[n++] = SplitPart{"cols", Mc, rn, A, transB ? b + Nc * ldb * esz : b + Nc * esz,
                          C ? C + Nc : nullptr, D + Nc};
  return n;
}

// Plan (and with a stream, launch) a call: one launch, or the parts of a
// split call (see plan_split) with their paths joined into one.
int plan_and_launch(int64_t M, int64_t N, int64_t K, int dtype, int transA, int transB,
                    float alpha, float beta, const void* A, int64_t lda, const void* B,
                    int64_t ldb, const float* C, int64_t ldc, const float* D, int64_t ldd,
                    bool launch, hipStream_t stream) {
  Plan plan;
  int st = plan_call(M, N, K, dtype, transA, transB, alpha, beta, A, lda, B, ldb, C, ldc, D, ldd,
                     plan);
  if (st != GEMM_OK) return st;
  SplitPart part[3];
  const int np = plan_split(M, N, dtype, transA, transB, A, lda, B, ldb, C, ldc, D, ldd, plan,
                            part);
  if (np > 0) {
    Plan pp[3];
    std::string path = "split";
    bool ok = true;
    for (int i = 0; i < np; ++i) {
      const SplitPart& q = part[i];
      st = plan_call(q.M, q.N, K, dtype, transA, transB, alpha, beta, q.A, lda, q.B, ldb, q.C,
                     ldc, q.D, ldd, pp[i]);
      if (st != GEMM_OK) return st;
      if (i == 0 && pp[0].tile != TILE_256x256) {  // the core missed the two-group kernel
        ok = false;
        break;
      }
      char head[96];
      std::snprintf(head, sizeof head, "%s %s %lldx%lld: ", i ? ";" : "", q.what, (long long)q.M,
                    (long long)q.N);
      path += head + current_path();
    }
    if (ok) {
      for (int i = 0; i < np && launch; ++i) {
        const hipError_t e = launch_plan(pp[i], dtype, transA, transB, stream);
        if (e != hipSuccess)
          return fail(GEMM_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
      }
      g_path = path;
      g_path_lazy = false;
      return GEMM_OK;
    }
    // one launch after all: plan the whole call again (it sets the path)
    st = plan_call(M, N, K, dtype, transA, transB, alpha, beta, A, lda, B, ldb, C, ldc, D, ldd,
                   plan);
    if (st != GEMM_OK) return st;
  }
  if (!launch) return GEMM_OK;
  const hipError_t e = launch_plan(plan, dtype, transA, transB, stream);
  if (e != hipSuccess)
    return fail(GEMM_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GEMM_OK;
}

void log_call(int64_t M, int64_t N, int64_t K, int status) {
  const char* lv = g_env.log;
  if (!lv || std::strcmp(lv, "debug") != 0) return;
  if (status == GEMM_OK)
    std::fprintf(stderr, "[gemm] M=%lld N=%lld K=%lld -> %s\n", (long long)M, (long long)N,
                 (long long)K, current_path().c_str());
  else
    std::fprintf(stderr, "[gemm] M=%lld N=%lld K=%lld -> error %d: %s\n", (long long)M,
                 (long long)N, (long long)K, status, g_err.c_str());
}

}  // namespace
}  // namespace dgt

extern "C" {

int gemm(int64_t M, int64_t N, int64_t K, int dtype, int transA, int transB, float alpha,
         float beta, const void* A, int64_t lda, const void* B, int64_t ldb, const float* C,
         int64_t ldc, float* D, int64_t ldd, void* stream) {
  const int st = dgt::plan_and_launch(M, N, K, dtype, transA, transB, alpha, beta, A, lda, B, ldb,
                                      C, ldc, D, ldd, true, static_cast<hipStream_t>(stream));
  dgt::log_call(M, N, K, st);
  return st;
}

int gemm_validate(int64_t M, int64_t N, int64_t K, int dtype, int transA, int transB, float alpha,
                  float beta, const void* A, int64_t lda, const void* B, int64_t ldb,
                  const float* C, int64_t ldc, const float* D, int64_t ldd) {
  const int st = dgt::plan_and_launch(M, N, K, dtype, transA, transB, alpha, beta, A, lda, B, ldb,
                                      C, ldc, D, ldd, false, nullptr);
  dgt::log_call(M, N, K, st);
  return st;
}

int gemm_i8(int64_t M, int64_t N, int64_t K, int transA, int transB, int32_t alpha, int32_t beta,
            const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const int32_t* C,
            int64_t ldc, int32_t* D, int64_t ldd, void* stream) {
  using namespace dgt;
  GemmByteArgs a;
  bool noop;
  int st = plan_i8(M, N, K, transA, transB, alpha, beta, A, lda, B, ldb, C, ldc, D, ldd, a, noop);
  if (st == GEMM_OK && !noop) {
    const hipError_t e =
        launch_byte(BYTE_I8, transA != 0, transB != 0, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      st = fail(GEMM_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  }
  log_call(M, N, K, st);
  return st;
}

int gemm_i8_validate(int64_t M, int64_t N, int64_t K, int transA, int transB, int32_t alpha,
                     int32_t beta, const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                     const int32_t* C, int64_t ldc, const int32_t* D, int64_t ldd) {
  dgt::GemmByteArgs a;
  bool noop;
  int st = dgt::plan_i8(M, N, K, transA, transB, alpha, beta, A, lda, B, ldb, C, ldc, D, ldd, a,
                        noop);
  dgt::log_call(M, N, K, st);
  return st;
}

const char* gemm_last_error(void) { return dgt::g_err.c_str(); }

const char* gemm_last_path(void) { return dgt::current_path().c_str(); }

int gemm_tile_order(int64_t tiles_m, int64_t tiles_n, int group_m, int32_t* tm, int32_t* tn) {
  if (tiles_m <= 0 || tiles_n <= 0 || group_m < 1 || !tm || !tn ||
      tiles_m * tiles_n > 0x7fffffff)
    return dgt::fail(GEMM_ERR_INVALID_ARG, "gemm_tile_order: bad arguments");
  const int total = (int)(tiles_m * tiles_n);
  for (int w = 0; w < total; ++w) {
    int m, n;
    dgt::schedule_tile(w, (int)tiles_m, (int)tiles_n, group_m, m, n);
    tm[w] = m;
    tn[w] = n;
  }
  return GEMM_OK;
}

}  // extern "C"
