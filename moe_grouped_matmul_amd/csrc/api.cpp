// C ABI of the library: argument validation, tile-configuration choice and
// launch on the caller's stream.  No allocation, no synchronisation, no host
// reads of device data, so every call can be captured into a hipGraph.

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "dg.h"
#include "dg_internal.hpp"

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_cu_cap{0};

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other; CU count cached alongside
std::atomic<int> g_dev_kind[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return DG_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks that a HIP device is current and is gfx950; returns its CU count (>0) or fails.
int check_device(int* cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(DG_ERR_DEVICE, "no HIP device available");
  }
  if (dev < kMaxDevices) {
    const int kind = g_dev_kind[dev].load(std::memory_order_acquire);
    if (kind == 1) {
      *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
      return DG_OK;
    }
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DG_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
  }
  const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) {
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_kind[dev].store(is950 ? 1 : 2, std::memory_order_release);
  }
  if (!is950) return fail(DG_ERR_DEVICE, "device %d is %s, this library is built for gfx950 only", dev, prop.gcnArchName);
  *cus = prop.multiProcessorCount;
  return DG_OK;
}

int effective_cus(int device_cus) {
  const int cap = g_cu_cap.load(std::memory_order_relaxed);
  return (cap > 0 && cap < device_cus) ? cap : device_cus;
}

int check_nk(int64_t N, int64_t K) {
  if (K <= 0 || K % 128 != 0) return fail(DG_ERR_SHAPE, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  if (N <= 0 || N % 16 != 0) return fail(DG_ERR_SHAPE, "N must be a positive multiple of 16 (got %lld)", (long long)N);
  if (K > (int64_t)1 << 30 || N > (int64_t)1 << 30) return fail(DG_ERR_SHAPE, "N or K too large");
  return DG_OK;
}

int check_operands(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb, const uint16_t* D) {
  if (!A || !sfa || !B || !sfb || !D) return fail(DG_ERR_INVALID_ARG, "null operand pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16))
    return fail(DG_ERR_ALIGN, "A, B and D must be 16-byte aligned");
  if (!aligned(sfa, 4) || !aligned(sfb, 4)) return fail(DG_ERR_ALIGN, "scale arrays must be 4-byte aligned");
  return DG_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Dense split-K plan: enough work items to cover the CUs twice when the
// output alone has too few tiles.  Splits never exceed the K blocks.
// 256 x 256 tiles (gemm_wide.hip, no K split) stream a third fewer operand
// bytes per flop than 256 x 128 ones; taken when they fill whole rounds of
// the CUs to at least 85%.
bool wide_fill(int64_t M, int64_t N, int cus) {
  if (M < 256 || N < 256) return false;
  const int64_t tw = ceil_div(M, 256) * ceil_div(N, 256);
  return (double)tw / (double)(ceil_div(tw, cus) * cus) >= 0.85;
}

// K-grouped form: 256 x 256 tiles of all groups where they fill whole rounds
// of the CUs to >= 85% (the dense rule), else 256 x 128 tiles.
bool kgrouped_wide(int64_t G, int64_t M, int64_t N, int cus) {
  const int64_t tw = G * ceil_div(M, 256) * ceil_div(N, 256);
  return M >= 256 && N >= 256 && tw <= ((int64_t)1 << 31) - 1 &&
         (double)tw / (double)(ceil_div(tw, cus) * cus) >= 0.85;
}

struct DensePlan {
  bool persist;  // persistent kernel (gemm_persist.hip), M > 128
  bool wide;     // wide-tile persistent kernel (gemm_wide.hip): 256 x 256 tiles, no K split
  int grid;      // persistent: workgroups
  int dp_tiles, sk_tiles, sk_pieces, sk_kb;
  bool lds;     // LDS-ring kernel (gemm_lds.hip)
  bool skinny;  // skinny kernel (gemm_skinny.hip), M <= 128
  int cfg;      // lds / v1 tile configuration, or skinny rows per tile (64 | 128)
  int wn;       // skinny: columns per wave (16 | 32)
  int m_tiles;
  int n_tiles;
  int splits;
  int kb_per_split;
};

// The LDS-ring kernel addresses operands with 32-bit buffer offsets.
bool fits_32bit(int64_t rows, int64_t N, int64_t K) {
  const int64_t lim = ((int64_t)1 << 32) - 1;
  return (rows + 256) * K < lim && (N + 256) * K < lim && rows * (K / 128) * 4 < lim;
}

// The persistent kernel addresses A, B, alpha and D of all groups with 32-bit
// buffer offsets and uses offsets from 0xFFFFFF00 up for lanes outside a tile.
bool fits_persistent(int64_t groups, int64_t rows, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)0xFFFFFF00 - 4096;
  return groups * (rows + 256) * K < lim && groups * (N + 256) * K < lim &&
         groups * (rows + 256) * (K / 128) * 4 < lim && groups * rows * N * 2 < lim;
}

// Persistent dense schedule over 256x128 tiles, one workgroup per CU: whole
// rounds of tiles; a partial last round is split along K into P <= 4 pieces
// run by the workgroups it would leave idle (when the workspace holds the
// partials), so every workgroup ends at about the same time.
void plan_persistent(DensePlan& pl, int64_t M, int64_t N, int64_t K, int cus, size_t ws_bytes) {
  const int KB = (int)(K / 128);
  const int64_t T = ceil_div(M, 256) * ceil_div(N, 128);
  pl.persist = true;
  pl.cfg = dg::kLds256x128;
  pl.m_tiles = (int)ceil_div(M, 256);
  pl.n_tiles = (int)ceil_div(N, 128);
  pl.splits = 1;
  pl.kb_per_split = KB;
  pl.dp_tiles = (int)T;
  pl.sk_tiles = 0;
  pl.sk_pieces = 1;
  pl.sk_kb = KB;
  pl.grid = (int)(T < cus ? T : cus);
  const int64_t rem = T < cus ? T : T % cus;
  if (rem == 0) return;
  int P = (int)(cus / rem);
  if (P > 4) P = 4;
  if (P > KB) P = KB;
  if (P < 2) return;
  const int kbs = (int)ceil_div(KB, P);
  P = (int)ceil_div(KB, kbs);  // every piece non-empty
  if (P < 2 || dg::persistent_workspace_bytes((int)rem, P) > ws_bytes ||
      dg::persistent_workspace_bytes((int)rem, P) > (size_t)0xFFFFFF00 - 4096)
    return;
  pl.dp_tiles = (int)(T - rem);
  pl.sk_tiles = (int)rem;
  pl.sk_pieces = P;
  pl.sk_kb = kbs;
  const int64_t g = T < cus ? rem * P : cus;
  pl.grid = (int)g;
}

// Skinny kernel (one workgroup per CU): column width and K split chosen so
// the workgroups fill the CUs in whole rounds.  Without a split the wider
// tile wins ties; with one, 16-column waves give the most tiles, and the split
// is at most K / (20 bm) (the fp32 partials then stay below a fifth of the
// weight bytes; more splits lose more in the fix-up than they gain), at most
// 16, and only as large as the workspace holds.
DensePlan plan_dense(int64_t M, int64_t N, int64_t K, int cus, size_t ws_bytes, bool allow_wide) {
  DensePlan pl;
  pl.persist = false;
  pl.wide = false;
  pl.grid = 0;
  pl.dp_tiles = pl.sk_tiles = 0;
  pl.sk_pieces = 1;
  pl.sk_kb = 0;
  pl.lds = false;
  pl.skinny = false;
  pl.wn = 0;
  const int KB = (int)(K / 128);
  if (M <= 128 && fits_32bit(M, N, K)) {
    pl.skinny = true;
    // 64 < M <= 128: one 128-row tile (weights read once) when the columns
    // alone nearly fill the CUs; otherwise two 64-row tiles, whose split-K
    // partials are half as large per tile
    pl.cfg = (M <= 64 || ceil_div(N, 64) < cus / 2) ? 64 : 128;
    pl.m_tiles = (int)ceil_div(M, pl.cfg);
    const int64_t t16 = pl.m_tiles * ceil_div(N, 64);
    const int64_t t32 = pl.m_tiles * ceil_div(N, 128);
    auto fill = [&](int64_t t) { return (double)t / (double)(ceil_div(t, cus) * cus); };
    pl.wn = (t16 >= cus && fill(t32) >= fill(t16)) ? 32 : 16;
    int cap_rows = pl.cfg;  // K split capped at K / (20 * cap_rows): partials (splits * bm * 4 B per column) <= K / 5
    // 64 < M <= 128 with two 64-row tiles: each streams all of A beside its
    // columns of B; one 128 x 128 tile halves those A reads, and wins where it
    // still fills the CUs through a K split (partials then up to K / 2.5 per column)
    if (M > 64 && pl.cfg == 64) {
      const int64_t t128 = ceil_div(N, 128);
      int64_t s128 = t128 < cus ? cus / t128 : 1;
      if (s128 > K / 1280) s128 = K / 1280;
      if (s128 > 16) s128 = 16;
      if (s128 >= 2 && (double)(t128 * s128) >= 0.85 * cus &&
          dg::skinny_workspace_bytes(128, 1, (int)t128, 32, (int)s128) <= ws_bytes) {
        pl.cfg = 128;
        pl.m_tiles = 1;
        pl.wn = 32;
        cap_rows = 64;
      }
    }
    pl.n_tiles = (int)ceil_div(N, 4 * pl.wn);
    const int64_t tiles = (int64_t)pl.m_tiles * pl.n_tiles;
    int splits = 1;
    if (tiles < cus) {
      splits = (int)(cus / tiles);
      const int cap = (int)(K / (20 * cap_rows));
      if (splits > cap) splits = cap;
      if (splits > 16) splits = 16;
      while (splits > 1 && (dg::skinny_workspace_bytes(pl.cfg, pl.m_tiles, pl.n_tiles, pl.wn, splits) > ws_bytes ||
                            dg::skinny_workspace_bytes(pl.cfg, pl.m_tiles, pl.n_tiles, pl.wn, splits) >
                                ((size_t)1 << 31)))
        --splits;
      if (splits < 2) splits = 1;
    }
    // whole ring cycles per split where that does not cost a split
    const int depth = dg::skinny_depth(pl.cfg, pl.wn);
    int kbs = (int)ceil_div(KB, splits);
    const int kbs_r = (int)ceil_div(kbs, depth) * depth;
    if (ceil_div(KB, kbs_r) == splits || kbs_r - kbs < depth / 2) kbs = kbs_r;
    pl.kb_per_split = kbs;
    pl.splits = (int)ceil_div(KB, pl.kb_per_split);
    return pl;
  }
  if (M > 128 && fits_persistent(1, M, N, K)) {
    const int64_t tw = ceil_div(M, 256) * ceil_div(N, 256);
    if (allow_wide && wide_fill(M, N, cus)) {
      pl.persist = true;
      pl.wide = true;
      pl.m_tiles = (int)ceil_div(M, 256);
      pl.n_tiles = (int)ceil_div(N, 256);
      pl.grid = (int)(tw < cus ? tw : cus);
      pl.splits = 1;
      pl.kb_per_split = KB;
      pl.dp_tiles = (int)tw;
      pl.sk_tiles = 0;
      pl.sk_pieces = 1;
      pl.sk_kb = KB;
      return pl;
    }
    plan_persistent(pl, M, N, K, cus, ws_bytes);
    return pl;
  }
  if (M > 128 && fits_32bit(M, N, K)) {
    pl.lds = true;
    pl.cfg = dg::kLds256x128;
    pl.m_tiles = (int)ceil_div(M, 256);
    pl.n_tiles = (int)ceil_div(N, 128);
    pl.splits = 1;
    pl.kb_per_split = (int)(K / 128);
    return pl;
  }
  pl.cfg = M <= 128 ? dg::kTile64x64 : dg::kTile128x128;
  const dg::TileShape ts = dg::tile_shape(pl.cfg);
  pl.m_tiles = (int)ceil_div(M, ts.bm);
  pl.n_tiles = (int)ceil_div(N, ts.bn);
  const int64_t tiles = (int64_t)pl.m_tiles * pl.n_tiles;
  int splits = 1;
  if (tiles < cus) {
    splits = (int)ceil_div(2 * (int64_t)cus, tiles);
    if (splits > KB) splits = KB;
    if (splits > 16) splits = 16;
    const size_t per_split = (size_t)M * (size_t)N * sizeof(float);
    const size_t fit = per_split ? ws_bytes / per_split : 0;
    if ((size_t)splits > fit) splits = (int)fit;
    if (splits < 2) splits = 1;
  }
  pl.kb_per_split = (int)ceil_div(KB, splits);
  pl.splits = (int)ceil_div(KB, pl.kb_per_split);
  return pl;
}

// Contiguous-form plan: the wide kernel (256 x 256 tiles) when K >= 4096,
// its tiles fill whole rounds of the CUs to >= 85% and each workgroup's tiles
// fit its pass table; else the persistent kernel over 128 x 256 tiles when
// that fits.
struct ContigPlan {
  bool wide;
  bool persist;
  int grid;
};
ContigPlan plan_contiguous(int64_t M_total, int64_t N, int64_t K, int64_t G, int cus) {
  ContigPlan cp{false, false, 0};
  const bool fits = fits_persistent(1, M_total, N, K) && fits_persistent(G, 0, N, K);
  const int64_t tw = ceil_div(M_total, 256) * ceil_div(N, 256);
  const int64_t gw = tw < cus ? tw : cus;
  // K >= 4096: with fewer K blocks per tile the second passes of tiles at
  // expert boundaries and the per-tile overheads outweigh the wider tile
  if (fits && M_total >= 256 && N >= 256 && K >= 4096 && ceil_div(tw, gw) <= dg::kWideMaxContigTiles &&
      (double)tw / (double)(ceil_div(tw, cus) * cus) >= 0.85) {
    cp.wide = true;
    cp.persist = true;
    cp.grid = (int)gw;
    return cp;
  }
  const int64_t ptiles = ceil_div(M_total, 128) * ceil_div(N, 256);
  const int pgrid = (int)(ptiles < cus ? ptiles : cus);
  cp.persist = fits && ceil_div(ptiles, pgrid) <= dg::kPersistentMaxContigTiles;
  cp.grid = pgrid;
  return cp;
}

}  // namespace

extern "C" {

int dg_fp8_gemm_nt(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb, uint16_t* D, int64_t M,
                   int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (M < 0) return fail(DG_ERR_SHAPE, "M must be >= 0 (got %lld)", (long long)M);
  if (M > ((int64_t)1 << 31) - 1) return fail(DG_ERR_SHAPE, "M too large");
  if (M == 0) return ok();
  if ((rc = check_operands(A, sfa, B, sfb, D))) return rc;
  if (workspace && (!aligned(workspace, 16) || workspace_bytes % 4))
    return fail(DG_ERR_WORKSPACE, "workspace must be 16-byte aligned with a size that is a multiple of 4");
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  const DensePlan pl = plan_dense(M, N, K, effective_cus(cus), workspace ? workspace_bytes : 0, true);
  dg::GemmParams p{};
  p.A = A;
  p.sfa = sfa;
  p.B = B;
  p.sfb = sfb;
  p.D = D;
  p.ws = static_cast<float*>(workspace);
  p.index = nullptr;
  p.rows = M;
  p.N = (int)N;
  p.K = (int)K;
  p.G = 1;
  p.m_tiles = pl.m_tiles;
  p.n_tiles = pl.n_tiles;
  p.splits = pl.splits;
  p.kb_per_split = pl.kb_per_split;
  p.dp_tiles = pl.dp_tiles;
  p.sk_tiles = pl.sk_tiles;
  p.sk_pieces = pl.sk_pieces;
  p.sk_kb = pl.sk_kb;
  if (std::getenv("DG_PRINT_CONFIGS") && pl.persist)
    std::fprintf(stderr,
                 "[dg] gemm_nt M=%lld N=%lld K=%lld kernel=%s grid=%d tiles=%d whole=%d tail=%d x %d pieces of %d\n",
                 (long long)M, (long long)N, (long long)K, pl.wide ? "wide" : "persistent", pl.grid,
                 pl.m_tiles * pl.n_tiles, pl.dp_tiles, pl.sk_tiles, pl.sk_pieces, pl.sk_kb);
  else if (std::getenv("DG_PRINT_CONFIGS"))
    std::fprintf(stderr, "[dg] gemm_nt M=%lld N=%lld K=%lld kernel=%s tile=%dx%d m_tiles=%d n_tiles=%d splits=%d\n",
                 (long long)M, (long long)N, (long long)K, pl.skinny ? "skinny" : (pl.lds ? "lds" : "v1"),
                 pl.skinny ? pl.cfg : (pl.lds ? dg::lds_tile_shape(pl.cfg).bm : dg::tile_shape(pl.cfg).bm),
                 pl.skinny ? 4 * pl.wn : (pl.lds ? dg::lds_tile_shape(pl.cfg).bn : dg::tile_shape(pl.cfg).bn),
                 pl.m_tiles, pl.n_tiles, pl.splits);
  hipError_t e;
  if (pl.wide)
    e = dg::launch_gemm_wide(dg::kDense, pl.grid, p, static_cast<hipStream_t>(stream));
  else if (pl.persist)
    e = dg::launch_gemm_persistent(dg::kDense, pl.grid, p, static_cast<hipStream_t>(stream));
  else if (pl.skinny)
    e = dg::launch_gemm_skinny(pl.cfg, pl.wn, p, static_cast<hipStream_t>(stream));
  else if (pl.lds)
    e = dg::launch_gemm_lds(dg::kDense, pl.cfg, p, static_cast<hipStream_t>(stream));
  else
    e = dg::launch_gemm(dg::kDense, pl.cfg, p, 1, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_fp8_gemm_nt_acc(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb, const float* C,
                       float* D, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (M < 0) return fail(DG_ERR_SHAPE, "M must be >= 0 (got %lld)", (long long)M);
  if (M > ((int64_t)1 << 31) - 1) return fail(DG_ERR_SHAPE, "M too large");
  if (M == 0) return ok();
  if (!A || !sfa || !B || !sfb || !D) return fail(DG_ERR_INVALID_ARG, "null operand pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || (C && !aligned(C, 16)))
    return fail(DG_ERR_ALIGN, "A, B, C and D must be 16-byte aligned");
  if (!aligned(sfa, 4) || !aligned(sfb, 4)) return fail(DG_ERR_ALIGN, "scale arrays must be 4-byte aligned");
  if (workspace && (!aligned(workspace, 16) || workspace_bytes % 4))
    return fail(DG_ERR_WORKSPACE, "workspace must be 16-byte aligned with a size that is a multiple of 4");
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  const int ecus = effective_cus(cus);
  DensePlan pl = plan_dense(M, N, K, ecus, workspace ? workspace_bytes : 0, false);
  if (!pl.persist && !pl.skinny) return fail(DG_ERR_SHAPE, "problem too large for the accumulating form");
  if (pl.persist && M * N * 4 >= (int64_t)0xFFFFFF00 - 4096)
    return fail(DG_ERR_SHAPE, "fp32 output too large for 32-bit buffer offsets");
  const bool wide = pl.persist && wide_fill(M, N, ecus);  // 256 x 256 tiles, no K split
  if (wide) {
    pl.m_tiles = (int)ceil_div(M, 256);
    pl.n_tiles = (int)ceil_div(N, 256);
    const int64_t tw = (int64_t)pl.m_tiles * pl.n_tiles;
    pl.grid = (int)(tw < ecus ? tw : ecus);
    pl.dp_tiles = (int)tw;
    pl.sk_tiles = 0;
    pl.sk_pieces = 1;
    pl.sk_kb = (int)(K / 128);
  }
  dg::GemmParams p{};
  p.A = A;
  p.sfa = sfa;
  p.B = B;
  p.sfb = sfb;
  p.Cacc = C;
  p.Dacc = D;
  p.ws = static_cast<float*>(workspace);
  p.rows = M;
  p.N = (int)N;
  p.K = (int)K;
  p.G = 1;
  p.m_tiles = pl.m_tiles;
  p.n_tiles = pl.n_tiles;
  p.splits = pl.splits;
  p.kb_per_split = pl.kb_per_split;
  p.dp_tiles = pl.dp_tiles;
  p.sk_tiles = pl.sk_tiles;
  p.sk_pieces = pl.sk_pieces;
  p.sk_kb = pl.sk_kb;
  if (std::getenv("DG_PRINT_CONFIGS"))
    std::fprintf(stderr, "[dg] gemm_nt_acc M=%lld N=%lld K=%lld kernel=%s\n", (long long)M, (long long)N, (long long)K,
                 wide ? "wide" : (pl.persist ? "persistent" : "skinny"));
  const hipError_t e =
      wide ? dg::launch_gemm_wide(dg::kDenseAcc, pl.grid, p, static_cast<hipStream_t>(stream))
           : (pl.persist ? dg::launch_gemm_persistent(dg::kDenseAcc, pl.grid, p, static_cast<hipStream_t>(stream))
                         : dg::launch_gemm_skinny(pl.cfg, pl.wn, p, static_cast<hipStream_t>(stream)));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_fp8_gemm_nt_ue8m0(const uint8_t* A, const int32_t* sfa, const uint8_t* B, const int32_t* sfb, uint16_t* D,
                         int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (M < 0) return fail(DG_ERR_SHAPE, "M must be >= 0 (got %lld)", (long long)M);
  if (M > ((int64_t)1 << 31) - 1) return fail(DG_ERR_SHAPE, "M too large");
  if (M == 0) return ok();
  if ((rc = check_operands(A, reinterpret_cast<const float*>(sfa), B, reinterpret_cast<const float*>(sfb), D)))
    return rc;
  if (workspace && (!aligned(workspace, 16) || workspace_bytes % 4))
    return fail(DG_ERR_WORKSPACE, "workspace must be 16-byte aligned with a size that is a multiple of 4");
  if (!fits_persistent(1, M, N, K)) return fail(DG_ERR_SHAPE, "problem too large for 32-bit buffer offsets");
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  DensePlan pl;
  const int ecus = effective_cus(cus);
  const bool wide = wide_fill(M, N, ecus);
  if (wide) {
    pl.m_tiles = (int)ceil_div(M, 256);
    pl.n_tiles = (int)ceil_div(N, 256);
    const int64_t tw = (int64_t)pl.m_tiles * pl.n_tiles;
    pl.grid = (int)(tw < ecus ? tw : ecus);
    pl.kb_per_split = (int)(K / 128);
    pl.dp_tiles = (int)tw;
    pl.sk_tiles = 0;
    pl.sk_pieces = 1;
    pl.sk_kb = (int)(K / 128);
  } else {
    plan_persistent(pl, M, N, K, ecus, workspace ? workspace_bytes : 0);
  }
  dg::GemmParams p{};
  p.A = A;
  p.sfa = reinterpret_cast<const float*>(sfa);  // packed UE8M0 words, read as such by the kernel
  p.B = B;
  p.sfb = reinterpret_cast<const float*>(sfb);
  p.D = D;
  p.ws = static_cast<float*>(workspace);
  p.rows = M;
  p.N = (int)N;
  p.K = (int)K;
  p.G = 1;
  p.m_tiles = pl.m_tiles;
  p.n_tiles = pl.n_tiles;
  p.splits = 1;
  p.kb_per_split = pl.kb_per_split;
  p.dp_tiles = pl.dp_tiles;
  p.sk_tiles = pl.sk_tiles;
  p.sk_pieces = pl.sk_pieces;
  p.sk_kb = pl.sk_kb;
  if (std::getenv("DG_PRINT_CONFIGS"))
    std::fprintf(stderr,
                 "[dg] gemm_nt_ue8m0 M=%lld N=%lld K=%lld kernel=%s grid=%d tiles=%d whole=%d tail=%d x %d pieces of %d\n",
                 (long long)M, (long long)N, (long long)K, wide ? "wide" : "persistent", pl.grid, pl.m_tiles * pl.n_tiles,
                 pl.dp_tiles, pl.sk_tiles, pl.sk_pieces, pl.sk_kb);
  const hipError_t e = wide ? dg::launch_gemm_wide(dg::kDenseUe8m0, pl.grid, p, static_cast<hipStream_t>(stream))
                            : dg::launch_gemm_persistent(dg::kDenseUe8m0, pl.grid, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_k_grouped_fp8_gemm_nt_contiguous(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb,
                                        const float* C, float* D, const int32_t* ks, int64_t G, int64_t M,
                                        int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (G < 1 || G > 1024) return fail(DG_ERR_SHAPE, "G must be in [1, 1024] (got %lld)", (long long)G);
  if (M < 0) return fail(DG_ERR_SHAPE, "M must be >= 0 (got %lld)", (long long)M);
  if (M > ((int64_t)1 << 31) - 1) return fail(DG_ERR_SHAPE, "M too large");
  if (M == 0) return ok();
  if (!A || !sfa || !B || !sfb || !D || !ks) return fail(DG_ERR_INVALID_ARG, "null operand pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || (C && !aligned(C, 16)))
    return fail(DG_ERR_ALIGN, "A, B, C and D must be 16-byte aligned");
  if (!aligned(sfa, 4) || !aligned(sfb, 4) || !aligned(ks, 4))
    return fail(DG_ERR_ALIGN, "scale arrays and ks must be 4-byte aligned");
  // one 256 x 128 tile grid per group over the shared operands; fp32 C and D
  // are addressed per group
  if (!fits_persistent(1, M, N, K) || (M + 256) * N * 4 >= (int64_t)0xFFFFFF00 - 4096)
    return fail(DG_ERR_SHAPE, "problem too large for 32-bit buffer offsets");
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  dg::GemmParams p{};
  p.A = A;
  p.sfa = sfa;
  p.B = B;
  p.sfb = sfb;
  p.Cacc = C;
  p.Dacc = D;
  p.index = ks;
  p.rows = M;
  p.N = (int)N;
  p.K = (int)K;
  p.G = (int)G;
  const int ecus = effective_cus(cus);
  const bool wide = kgrouped_wide(G, M, N, ecus);
  p.m_tiles = (int)ceil_div(M, 256);
  p.n_tiles = (int)ceil_div(N, wide ? 256 : 128);
  p.splits = 1;
  p.kb_per_split = (int)(K / 128);
  p.dp_tiles = 0;
  p.sk_tiles = 0;
  p.sk_pieces = 1;
  p.sk_kb = (int)(K / 128);
  const int64_t tiles = G * p.m_tiles * p.n_tiles;
  if (tiles > ((int64_t)1 << 31) - 1) return fail(DG_ERR_SHAPE, "too many tiles");
  const int grid = (int)(tiles < ecus ? tiles : ecus);
  if (std::getenv("DG_PRINT_CONFIGS"))
    std::fprintf(stderr, "[dg] k_grouped G=%lld M=%lld N=%lld K=%lld kernel=%s tiles=%lld grid=%d\n", (long long)G,
                 (long long)M, (long long)N, (long long)K, wide ? "wide" : "persistent", (long long)tiles, grid);
  const hipError_t e = wide ? dg::launch_gemm_wide(dg::kKGrouped, grid, p, static_cast<hipStream_t>(stream))
                            : dg::launch_gemm_persistent(dg::kKGrouped, grid, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_bf16_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* D, int64_t M, int64_t N, int64_t K,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (K <= 0 || K % 64 != 0) return fail(DG_ERR_SHAPE, "K must be a positive multiple of 64 (got %lld)", (long long)K);
  if (N <= 0 || N % 16 != 0) return fail(DG_ERR_SHAPE, "N must be a positive multiple of 16 (got %lld)", (long long)N);
  if (K > (int64_t)1 << 29 || N > (int64_t)1 << 30) return fail(DG_ERR_SHAPE, "N or K too large");
  if (M < 0) return fail(DG_ERR_SHAPE, "M must be >= 0 (got %lld)", (long long)M);
  if (M > ((int64_t)1 << 31) - 1) return fail(DG_ERR_SHAPE, "M too large");
  if (M == 0) return ok();
  if (!A || !B || !D) return fail(DG_ERR_INVALID_ARG, "null operand pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16))
    return fail(DG_ERR_ALIGN, "A, B and D must be 16-byte aligned");
  if (workspace && (!aligned(workspace, 16) || workspace_bytes % 4))
    return fail(DG_ERR_WORKSPACE, "workspace must be 16-byte aligned with a size that is a multiple of 4");
  int rc = 0;
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  // the persistent kernels' schedule over K blocks of 128 bytes (64 bf16)
  if (!fits_persistent(1, M, N, 2 * K)) return fail(DG_ERR_SHAPE, "problem too large for 32-bit buffer offsets");
  DensePlan pl;
  const int ecus = effective_cus(cus);
  const bool wide = wide_fill(M, N, ecus);
  if (wide) {
    pl.m_tiles = (int)ceil_div(M, 256);
    pl.n_tiles = (int)ceil_div(N, 256);
    const int64_t tw = (int64_t)pl.m_tiles * pl.n_tiles;
    pl.grid = (int)(tw < ecus ? tw : ecus);
    pl.kb_per_split = (int)(2 * K / 128);
    pl.dp_tiles = (int)tw;
    pl.sk_tiles = 0;
    pl.sk_pieces = 1;
    pl.sk_kb = pl.kb_per_split;
  } else {
    plan_persistent(pl, M, N, 2 * K, ecus, workspace ? workspace_bytes : 0);
  }
  dg::GemmParams p{};
  p.A = reinterpret_cast<const uint8_t*>(A);
  p.B = reinterpret_cast<const uint8_t*>(B);
  p.D = D;
  p.ws = static_cast<float*>(workspace);
  p.rows = M;
  p.N = (int)N;
  p.K = (int)K;  // elements; the kernel addresses rows of 2 K bytes
  p.G = 1;
  p.m_tiles = pl.m_tiles;
  p.n_tiles = pl.n_tiles;
  p.splits = 1;
  p.kb_per_split = pl.kb_per_split;
  p.dp_tiles = pl.dp_tiles;
  p.sk_tiles = pl.sk_tiles;
  p.sk_pieces = pl.sk_pieces;
  p.sk_kb = pl.sk_kb;
  if (std::getenv("DG_PRINT_CONFIGS"))
    std::fprintf(stderr,
                 "[dg] bf16_gemm_nt M=%lld N=%lld K=%lld kernel=%s grid=%d tiles=%d whole=%d tail=%d x %d pieces of %d\n",
                 (long long)M, (long long)N, (long long)K, wide ? "wide" : "persistent", pl.grid, pl.m_tiles * pl.n_tiles,
                 pl.dp_tiles, pl.sk_tiles, pl.sk_pieces, pl.sk_kb);
  const hipError_t e = wide ? dg::launch_gemm_wide(dg::kDenseBf16, pl.grid, p, static_cast<hipStream_t>(stream))
                            : dg::launch_gemm_persistent(dg::kDenseBf16, pl.grid, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb,
                                        uint16_t* D, const int32_t* m_indices, int64_t M_total, int64_t N,
                                        int64_t K, int64_t G, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (M_total < 0) return fail(DG_ERR_SHAPE, "M_total must be >= 0");
  if (M_total > ((int64_t)1 << 31) - 1) return fail(DG_ERR_SHAPE, "M_total too large");
  if (G < 1 || G > 65536) return fail(DG_ERR_SHAPE, "G must be in [1, 65536] (got %lld)", (long long)G);
  if (M_total == 0) return ok();
  if ((rc = check_operands(A, sfa, B, sfb, D))) return rc;
  if (!m_indices) return fail(DG_ERR_INVALID_ARG, "null m_indices");
  if (!aligned(m_indices, 4)) return fail(DG_ERR_ALIGN, "m_indices must be 4-byte aligned");
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  // 256 x 256 tiles (wide kernel, two passes where a tile straddles two
  // experts) when they fill whole rounds of the CUs to >= 85%; otherwise
  // 128 x 256 tiles, each inside one 128-row aligned expert segment.  Both
  // need their 32-bit offsets to fit and each workgroup's tiles to fit its
  // table.
  const int ecus = effective_cus(cus);
  const ContigPlan cp = plan_contiguous(M_total, N, K, G, ecus);
  const int64_t ptiles = ceil_div(M_total, 128) * ceil_div(N, 256);
  const int pgrid = (int)(ptiles < ecus ? ptiles : ecus);
  const bool persist = cp.persist;
  const bool lds = persist || fits_32bit(M_total, N, K);
  const int bm = 128;
  const int bn = lds ? 256 : 128;
  dg::GemmParams p{};
  p.A = A;
  p.sfa = sfa;
  p.B = B;
  p.sfb = sfb;
  p.D = D;
  p.index = m_indices;
  p.rows = M_total;
  p.N = (int)N;
  p.K = (int)K;
  p.G = (int)G;
  p.m_tiles = (int)ceil_div(M_total, bm);
  p.n_tiles = (int)ceil_div(N, bn);
  p.splits = 1;
  p.kb_per_split = (int)(K / 128);
  if (std::getenv("DG_PRINT_CONFIGS"))
    std::fprintf(stderr, "[dg] contiguous M_total=%lld N=%lld K=%lld G=%lld tile=%dx%d kernel=%s\n", (long long)M_total,
                 (long long)N, (long long)K, (long long)G, cp.wide ? 256 : bm, bn,
                 cp.wide ? "wide" : (persist ? "persistent" : "grid"));
  hipError_t e;
  if (cp.wide) {
    p.m_tiles = (int)ceil_div(M_total, 256);
    p.n_tiles = (int)ceil_div(N, 256);
    e = dg::launch_gemm_wide(dg::kContiguous, cp.grid, p, static_cast<hipStream_t>(stream));
  } else if (persist) {
    p.dp_tiles = (int)ptiles;  // every tile whole: no K-split tail, no workspace
    p.sk_tiles = 0;
    p.sk_pieces = 1;
    p.sk_kb = (int)(K / 128);
    e = dg::launch_gemm_persistent(dg::kContiguous, pgrid, p, static_cast<hipStream_t>(stream));
  } else if (lds) {
    e = dg::launch_gemm_lds(dg::kContiguous, dg::kLds128x256, p, static_cast<hipStream_t>(stream));
  } else {
    e = dg::launch_gemm(dg::kContiguous, dg::kTile128x128, p, 1, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_m_grouped_fp8_gemm_nt_masked(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb,
                                    uint16_t* D, const int32_t* masked_m, int64_t G, int64_t max_m, int64_t N,
                                    int64_t K, int64_t expected_m, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (G < 1 || G > 65536) return fail(DG_ERR_SHAPE, "G must be in [1, 65536] (got %lld)", (long long)G);
  if (max_m < 0) return fail(DG_ERR_SHAPE, "max_m must be >= 0");
  if (G * max_m > ((int64_t)1 << 31) - 1) return fail(DG_ERR_SHAPE, "G * max_m too large");
  if (max_m == 0) return ok();
  if ((rc = check_operands(A, sfa, B, sfb, D))) return rc;
  if (!masked_m) return fail(DG_ERR_INVALID_ARG, "null masked_m");
  if (!aligned(masked_m, 4)) return fail(DG_ERR_ALIGN, "masked_m must be 4-byte aligned");
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  (void)expected_m;
  // persistent kernel with a device-side task list over the active tiles
  const bool persist = G <= 1024 && fits_persistent(G, max_m, N, K);
  const bool lds = persist || fits_32bit(max_m, N, K);
  const int cfg = lds ? (int)dg::kLds256x128 : (max_m <= 64 ? dg::kTile64x128 : dg::kTile128x128);
  const dg::TileShape ts = lds ? dg::lds_tile_shape(cfg) : dg::tile_shape(cfg);
  dg::GemmParams p{};
  p.A = A;
  p.sfa = sfa;
  p.B = B;
  p.sfb = sfb;
  p.D = D;
  p.index = masked_m;
  p.rows = max_m;
  p.N = (int)N;
  p.K = (int)K;
  p.G = (int)G;
  // the persistent kernel runs 128 x 256 tiles
  p.m_tiles = (int)ceil_div(max_m, persist ? 128 : ts.bm);
  p.n_tiles = (int)ceil_div(N, persist ? 256 : ts.bn);
  p.splits = 1;
  p.kb_per_split = (int)(K / 128);
  if (std::getenv("DG_PRINT_CONFIGS"))
    std::fprintf(stderr, "[dg] masked G=%lld max_m=%lld N=%lld K=%lld tile=%dx%d kernel=%s\n", (long long)G,
                 (long long)max_m, (long long)N, (long long)K, persist ? 128 : ts.bm, persist ? 256 : ts.bn,
                 persist ? "persistent" : "grid");
  hipError_t e;
  if (persist) {
    const int64_t tiles = G * p.m_tiles * p.n_tiles;
    const int ecus = effective_cus(cus);
    e = dg::launch_gemm_persistent(dg::kMasked, (int)(tiles < ecus ? tiles : ecus), p,
                                   static_cast<hipStream_t>(stream));
  } else if (lds) {
    e = dg::launch_gemm_lds(dg::kMasked, cfg, p, static_cast<hipStream_t>(stream));
  } else {
    e = dg::launch_gemm(dg::kMasked, cfg, p, (int)G, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_quant_1x128(const float* x, uint8_t* q, float* sfa, int64_t G, int64_t M, int64_t K, void* stream) {
  if (K <= 0 || K % 128) return fail(DG_ERR_SHAPE, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  if (G < 0 || M < 0) return fail(DG_ERR_SHAPE, "G and M must be >= 0");
  if (G > ((int64_t)1 << 31) || M > ((int64_t)1 << 31) || G * M * (K / 128) > ((int64_t)1 << 35))
    return fail(DG_ERR_SHAPE, "problem too large");
  if (G == 0 || M == 0) return ok();
  if (!x || !q || !sfa) return fail(DG_ERR_INVALID_ARG, "null pointer");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(DG_ERR_ALIGN, "x and q must be 16-byte aligned");
  if (!aligned(sfa, 4)) return fail(DG_ERR_ALIGN, "sfa must be 4-byte aligned");
  int cus = 0;
  int rc = check_device(&cus);
  if (rc) return rc;
  const hipError_t e = dg::launch_quant_1x128(x, q, sfa, G, M, K, false, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_quant_128x128(const float* x, uint8_t* q, float* sfb, int64_t G, int64_t N, int64_t K, void* stream) {
  if (K <= 0 || K % 128) return fail(DG_ERR_SHAPE, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  if (G < 0 || N < 0) return fail(DG_ERR_SHAPE, "G and N must be >= 0");
  if (G > ((int64_t)1 << 31) || N > ((int64_t)1 << 31) || G * ceil_div(N, 128) * (K / 128) > ((int64_t)1 << 31) - 1)
    return fail(DG_ERR_SHAPE, "problem too large");
  if (G == 0 || N == 0) return ok();
  if (!x || !q || !sfb) return fail(DG_ERR_INVALID_ARG, "null pointer");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(DG_ERR_ALIGN, "x and q must be 16-byte aligned");
  if (!aligned(sfb, 4)) return fail(DG_ERR_ALIGN, "sfb must be 4-byte aligned");
  int cus = 0;
  int rc = check_device(&cus);
  if (rc) return rc;
  const hipError_t e = dg::launch_quant_128x128(x, q, sfb, G, N, K, false, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_quant_1x128_ue8m0(const float* x, uint8_t* q, int32_t* sfa, int64_t G, int64_t M, int64_t K, void* stream) {
  if (K <= 0 || K % 128) return fail(DG_ERR_SHAPE, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  if (G < 0 || M < 0) return fail(DG_ERR_SHAPE, "G and M must be >= 0");
  if (G > ((int64_t)1 << 31) || M > ((int64_t)1 << 31) || G * M * (K / 128) > ((int64_t)1 << 35))
    return fail(DG_ERR_SHAPE, "problem too large");
  if (G == 0 || M == 0) return ok();
  if (!x || !q || !sfa) return fail(DG_ERR_INVALID_ARG, "null pointer");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(DG_ERR_ALIGN, "x and q must be 16-byte aligned");
  if (!aligned(sfa, 4)) return fail(DG_ERR_ALIGN, "sfa must be 4-byte aligned");
  int cus = 0;
  int rc = check_device(&cus);
  if (rc) return rc;
  const hipError_t e = dg::launch_quant_1x128(x, q, sfa, G, M, K, true, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_quant_128x128_ue8m0(const float* x, uint8_t* q, int32_t* sfb, int64_t G, int64_t N, int64_t K, void* stream) {
  if (K <= 0 || K % 128) return fail(DG_ERR_SHAPE, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  if (G < 0 || N < 0) return fail(DG_ERR_SHAPE, "G and N must be >= 0");
  if (G > ((int64_t)1 << 31) || N > ((int64_t)1 << 31) || G * ceil_div(N, 128) * (K / 128) > ((int64_t)1 << 31) - 1)
    return fail(DG_ERR_SHAPE, "problem too large");
  if (G == 0 || N == 0) return ok();
  if (!x || !q || !sfb) return fail(DG_ERR_INVALID_ARG, "null pointer");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(DG_ERR_ALIGN, "x and q must be 16-byte aligned");
  if (!aligned(sfb, 4)) return fail(DG_ERR_ALIGN, "sfb must be 4-byte aligned");
  int cus = 0;
  int rc = check_device(&cus);
  if (rc) return rc;
  const hipError_t e = dg::launch_quant_128x128(x, q, sfb, G, N, K, true, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t dg_get_workspace_size(int op, int64_t rows, int64_t N, int64_t K, int64_t G) {
  (void)G;
  if (op != DG_OP_GEMM_NT && op != DG_OP_BF16_GEMM_NT && op != DG_OP_GEMM_NT_UE8M0) return 0;
  if (rows <= 0 || N <= 0 || K <= 0 || K % (op == DG_OP_BF16_GEMM_NT ? 64 : 128)) return 0;
  int cus = 0;
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
  }
  (void)hipGetLastError();
  if (cus <= 0) cus = 256;
  if ((op == DG_OP_GEMM_NT_UE8M0 || op == DG_OP_BF16_GEMM_NT) && wide_fill(rows, N, effective_cus(cus)))
    return 0;  // 256 x 256 tiles, no split
  if (op == DG_OP_BF16_GEMM_NT || op == DG_OP_GEMM_NT_UE8M0) {
    const int64_t kb = op == DG_OP_BF16_GEMM_NT ? 2 * K : K;  // bytes per operand row
    if (!fits_persistent(1, rows, N, kb)) return 0;
    DensePlan pb;
    plan_persistent(pb, rows, N, kb, effective_cus(cus), (size_t)-1);
    return (dg::persistent_workspace_bytes(pb.sk_tiles, pb.sk_pieces) + 15) / 16 * 16;
  }
  // sized for the 256 x 128 plan, which the accumulating form also uses where
  // 256 x 256 tiles do not apply (those need no workspace; a larger one is unused)
  const DensePlan pl = plan_dense(rows, N, K, effective_cus(cus), (size_t)-1, false);
  if (pl.persist) return (dg::persistent_workspace_bytes(pl.sk_tiles, pl.sk_pieces) + 15) / 16 * 16;
  if (pl.splits <= 1) return 0;
  if (pl.skinny)
    return (dg::skinny_workspace_bytes(pl.cfg, pl.m_tiles, pl.n_tiles, pl.wn, pl.splits) + 15) / 16 * 16;
  return (size_t)pl.splits * (size_t)rows * (size_t)N * sizeof(float);
}

const char* dg_describe_plan(int op, int64_t rows, int64_t N, int64_t K, int64_t G) {
  (void)G;
  thread_local std::string text;
  text.clear();
  if ((op != DG_OP_GEMM_NT && op != DG_OP_CONTIGUOUS && op != DG_OP_GEMM_NT_UE8M0 && op != DG_OP_BF16_GEMM_NT &&
       op != DG_OP_K_GROUPED) ||
      rows <= 0 || N <= 0 || K <= 0 || K % (op == DG_OP_BF16_GEMM_NT ? 64 : 128) || N % 16)
    return text.c_str();
  int cus = 0;
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
  }
  (void)hipGetLastError();
  if (cus <= 0) cus = 256;
  char buf[256];
  if (op == DG_OP_CONTIGUOUS) {
    const ContigPlan cp = plan_contiguous(rows, N, K, G < 1 ? 1 : G, effective_cus(cus));
    std::snprintf(buf, sizeof(buf), "kernel=%s tile=%dx256 grid=%d", cp.wide ? "wide" : (cp.persist ? "persistent" : "grid"),
                  cp.wide ? 256 : 128, cp.grid);
    text = buf;
    return text.c_str();
  }
  if (op == DG_OP_K_GROUPED) {
    const int64_t g = G < 1 ? 1 : G;
    const int ecus = effective_cus(cus);
    const bool wide = kgrouped_wide(g, rows, N, ecus);
    const int64_t tiles = g * ceil_div(rows, 256) * ceil_div(N, wide ? 256 : 128);
    std::snprintf(buf, sizeof(buf), "kernel=%s tile=256x%d grid=%lld tiles=%lld", wide ? "wide" : "persistent",
                  wide ? 256 : 128, (long long)(tiles < ecus ? tiles : ecus), (long long)tiles);
    text = buf;
    return text.c_str();
  }
  if (op == DG_OP_GEMM_NT_UE8M0 || op == DG_OP_BF16_GEMM_NT) {
    const int ecus = effective_cus(cus);
    const int64_t kbytes = op == DG_OP_BF16_GEMM_NT ? 2 * K : K;  // bytes per operand row
    if (wide_fill(rows, N, ecus)) {
      const int64_t tw = ceil_div(rows, 256) * ceil_div(N, 256);
      std::snprintf(buf, sizeof(buf), "kernel=wide tile=256x256 grid=%d tiles=%d whole=%d tail=0x1",
                    (int)(tw < ecus ? tw : ecus), (int)tw, (int)tw);
    } else if (fits_persistent(1, rows, N, kbytes)) {
      DensePlan pb;
      plan_persistent(pb, rows, N, kbytes, ecus, (size_t)-1);
      std::snprintf(buf, sizeof(buf), "kernel=persistent tile=256x128 grid=%d tiles=%d whole=%d tail=%dx%d", pb.grid,
                    pb.m_tiles * pb.n_tiles, pb.dp_tiles, pb.sk_tiles, pb.sk_pieces);
    } else {
      buf[0] = 0;
    }
    text = buf;
    return text.c_str();
  }
  const DensePlan pl = plan_dense(rows, N, K, effective_cus(cus), (size_t)-1, true);
  if (pl.wide || pl.persist)
    std::snprintf(buf, sizeof(buf), "kernel=%s tile=%dx%d grid=%d tiles=%d whole=%d tail=%dx%d",
                  pl.wide ? "wide" : "persistent", 256, pl.wide ? 256 : 128, pl.grid, pl.m_tiles * pl.n_tiles,
                  pl.dp_tiles, pl.sk_tiles, pl.sk_pieces);
  else if (pl.skinny)
    std::snprintf(buf, sizeof(buf), "kernel=skinny tile=%dx%d tiles=%d splits=%d", pl.cfg, 4 * pl.wn,
                  pl.m_tiles * pl.n_tiles, pl.splits);
  else
    std::snprintf(buf, sizeof(buf), "kernel=%s tiles=%d splits=%d", pl.lds ? "lds" : "v1", pl.m_tiles * pl.n_tiles,
                  pl.splits);
  text = buf;
  return text.c_str();
}

int dg_get_m_alignment_for_contiguous_layout(void) { return 128; }

int dg_set_num_cus(int n) {
  g_cu_cap.store(n > 0 ? n : 0, std::memory_order_relaxed);
  return ok();
}

int dg_get_num_cus(void) {
  int dev = -1;
  int cus = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
  }
  (void)hipGetLastError();
  if (cus <= 0) return 0;
  return effective_cus(cus);
}

const char* dg_get_last_error(void) { return g_last_error.c_str(); }

const char* dg_version(void) { return "dg-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
