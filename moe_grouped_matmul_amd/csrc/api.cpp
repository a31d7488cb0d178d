// C ABI of the library: argument validation, tile-configuration choice and
// launch on the caller's stream.  No allocation, no synchronisation, no host
// reads of device data, so every call can be captured into a hipGraph.
//
// The kernels address one launch's activations, scales and outputs, and one
// expert's weights, with 32-bit byte offsets from 64-bit bases.  A call whose
// rows would not fit is split into row chunks launched back to back on the
// same stream (each chunk its own plan; chunks that share a split-K
// workspace run in stream order, and every launch leaves its counters at
// zero).  Only weights of 4 GiB or more per expert, more than 1024 groups
// and the K-grouped form past 32-bit offsets are rejected (DG_ERR_SHAPE).
//
// DG_FORCE_CONFIG (debug, read on every call): a comma-separated list of
//   kernel=wide|persistent  force the 256x256 or the 256x128 / 128x256 tile
//                           kernel where the planner chooses between them
//                           (rows > 128 outside the skinny domain, or the
//                           contiguous form)
//   chunk_rows=<n>          at most n rows per launch (rounded down to a
//                           multiple of 256, at least 256)
//   skinny=<bm>x<wn>x<s>x<p>  rows <= 2048: bm-row tiles (64 | 128) of 4 wn
//                           columns (wn 16 | 32), K split s ways (bounded by
//                           the K blocks and the workspace), ring depth p
//                           among the compiled ones (dg::skinny_depth_ok)
// DG_PRINT_CONFIGS (debug): print each launch's plan on stderr.
// DG_CHECK_LAYOUT (debug): the contiguous forms copy m_indices to the host
// (synchronising the stream; skipped while the stream is being captured) and
// reject a layout in which an aligned 128-row block holds rows of two
// experts (DG_ERR_INVALID_ARG).

#include <algorithm>
#include <atomic>
#include <vector>
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

// Byte offsets a kernel may use inside one buffer range: below the
// out-of-range marker (0xFFFFFF00) the kernels give lanes outside a tile.
constexpr int64_t kOffLim = (int64_t)0xFFFFFF00 - 4096;
constexpr int64_t kMaxGroups = 1024;

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

// CU count of the current device for the planning queries (256, the
// MI355X's, when no device is visible).
int query_cus() {
  int cus = 0;
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
  }
  (void)hipGetLastError();
  return cus > 0 ? cus : 256;
}

int effective_cus(int device_cus) {
  const int cap = g_cu_cap.load(std::memory_order_relaxed);
  return (cap > 0 && cap < device_cus) ? cap : device_cus;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- DG_FORCE_CONFIG
enum ForceKernel { kForceNone = 0, kForceWide = 1, kForcePersistent = 2 };
struct Force {
  int kernel = kForceNone;
  int64_t chunk_rows = 0;
  int sk_bm = 0, sk_wn = 0, sk_splits = 0, sk_depth = 0;  // skinny=<bm>x<wn>x<s>x<p>
};
Force forced() {
  Force f;
  const char* e = std::getenv("DG_FORCE_CONFIG");
  if (!e) return f;
  std::string s(e);
  size_t pos = 0;
  while (pos <= s.size()) {
    size_t end = s.find(',', pos);
    if (end == std::string::npos) end = s.size();
    const std::string item = s.substr(pos, end - pos);
    if (item == "kernel=wide") f.kernel = kForceWide;
    else if (item == "kernel=persistent") f.kernel = kForcePersistent;
    else if (item.rfind("chunk_rows=", 0) == 0) f.chunk_rows = std::atoll(item.c_str() + 11);
    else if (item.rfind("skinny=", 0) == 0) {
      int bm = 0, wn = 0, sp = 0, d = 0;
      if (std::sscanf(item.c_str() + 7, "%dx%dx%dx%d", &bm, &wn, &sp, &d) == 4 && (bm == 64 || bm == 128) &&
          (wn == 16 || wn == 32) && sp >= 1 && dg::skinny_depth_ok(bm, wn, d)) {
        f.sk_bm = bm;
        f.sk_wn = wn;
        f.sk_splits = sp;
        f.sk_depth = d;
      }
    }
    pos = end + 1;
  }
  return f;
}
bool print_configs() { return std::getenv("DG_PRINT_CONFIGS") != nullptr; }

// Rows per launch (a multiple of 256): A rows of row_bytes each (plus one
// tile of overhang) and output rows of out_bytes each stay inside 32-bit
// offsets; 0 when not even 256 rows fit.
int64_t launch_rows(int64_t row_bytes, int64_t out_bytes) {
  int64_t r = std::min(kOffLim / row_bytes - 256, kOffLim / out_bytes);
  const Force f = forced();
  if (f.chunk_rows > 0 && f.chunk_rows < r) r = std::max<int64_t>(f.chunk_rows, 256);
  r = r / 256 * 256;
  return r >= 256 ? r : 0;
}

int check_nk(int64_t N, int64_t K) {
  if (K <= 0 || K % 128 != 0) return fail(DG_ERR_SHAPE, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  if (N <= 0 || N % 16 != 0) return fail(DG_ERR_SHAPE, "N must be a positive multiple of 16 (got %lld)", (long long)N);
  if (K > (int64_t)1 << 30 || N > (int64_t)1 << 30) return fail(DG_ERR_SHAPE, "N or K too large");
  return DG_OK;
}

// One expert's weights (N rows of row_bytes, plus one tile of overhang) must
// fit 32-bit offsets; the caller's activation scales too (rows x K/128 x 4 B).
int check_weights_and_scales(int64_t N, int64_t row_bytes, int64_t rows, int64_t KB) {
  if ((N + 256) * row_bytes >= kOffLim)
    return fail(DG_ERR_SHAPE, "weights of %lld x %lld bytes per expert exceed 4 GiB", (long long)N, (long long)row_bytes);
  if (rows * KB * 4 >= kOffLim) return fail(DG_ERR_SHAPE, "activation scales exceed 4 GiB");
  return DG_OK;
}

int check_operands(const void* A, const void* sfa, const void* B, const void* sfb, const void* D) {
  if (!A || !sfa || !B || !sfb || !D) return fail(DG_ERR_INVALID_ARG, "null operand pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16))
    return fail(DG_ERR_ALIGN, "A, B and D must be 16-byte aligned");
  if (!aligned(sfa, 4) || !aligned(sfb, 4)) return fail(DG_ERR_ALIGN, "scale arrays must be 4-byte aligned");
  return DG_OK;
}

int check_workspace(const void* ws, size_t bytes) {
  if (ws && (!aligned(ws, 16) || bytes % 4))
    return fail(DG_ERR_WORKSPACE, "workspace must be 16-byte aligned with a size that is a multiple of 4");
  return DG_OK;
}

// 256 x 256 tiles (gemm_wide.hip, no K split) stream a third fewer operand
// bytes per flop than 256 x 128 ones; taken when they fill whole rounds of
// the CUs to at least 85%, and for the FP8 forms also when they make one
// round on at least 60% of the CUs: measured 14-22% faster there than 256 x
// 128 tiles with a K-split tail at K = 4096-7168 and 1.3-1.9x faster at K =
// 1024-2048, on the fp8, accumulating and UE8M0 forms; at 56% the two were
// within the spread between boxes, and the BF16 form was not faster below
// 85%.
bool wide_fill(int64_t M, int64_t N, int cus, bool fp8) {
  if (M < 256 || N < 256) return false;
  const int64_t tw = ceil_div(M, 256) * ceil_div(N, 256);
  if (fp8 && tw <= cus && (double)tw >= 0.6 * (double)cus) return true;
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
  bool wide = false;    // wide-tile persistent kernel (gemm_wide.hip): 256 x 256 tiles, no K split
  bool persist = false; // persistent kernel (gemm_persist.hip): 256 x 128 tiles, K-split tail
  bool skinny = false;  // skinny kernel (gemm_skinny.hip), M <= 2048
  int grid = 0;         // wide / persistent: workgroups
  int dp_tiles = 0, sk_tiles = 0, sk_pieces = 1, sk_kb = 0;
  int cfg = 0;          // skinny rows per tile (64 | 128)
  int wn = 0;           // skinny: columns per wave (16 | 32)
  int depth = 0;        // skinny: ring depth
  int m_tiles = 0;
  int n_tiles = 0;
  int splits = 1;
  int kb_per_split = 0;
};

// Wide plan: every tile whole, one workgroup per CU (K = blocks of 128 bytes).
void plan_wide(DensePlan& pl, int64_t M, int64_t N, int64_t kbytes, int cus) {
  pl.wide = true;
  pl.persist = true;
  pl.m_tiles = (int)ceil_div(M, 256);
  pl.n_tiles = (int)ceil_div(N, 256);
  const int64_t tw = (int64_t)pl.m_tiles * pl.n_tiles;
  pl.grid = (int)(tw < cus ? tw : cus);
  pl.splits = 1;
  pl.kb_per_split = (int)(kbytes / 128);
  pl.dp_tiles = (int)tw;
  pl.sk_tiles = 0;
  pl.sk_pieces = 1;
  pl.sk_kb = pl.kb_per_split;
}

// Persistent dense schedule over 256x128 tiles, one workgroup per CU: whole
// rounds of tiles; a partial last round is split along K into P <= 4 pieces
// run by the workgroups it would leave idle (when the workspace holds the
// partials), so every workgroup ends at about the same time.  K counts
// bytes per operand row (128 per block).
void plan_persistent(DensePlan& pl, int64_t M, int64_t N, int64_t K, int cus, size_t ws_bytes) {
  const int KB = (int)(K / 128);
  const int64_t T = ceil_div(M, 256) * ceil_div(N, 128);
  pl.wide = false;
  pl.persist = true;
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
  if (P < 2 || rem > dg::kWsMaxCounters || dg::persistent_workspace_bytes((int)rem, P) > ws_bytes ||
      dg::persistent_workspace_bytes((int)rem, P) > (size_t)kOffLim)
    return;
  pl.dp_tiles = (int)(T - rem);
  pl.sk_tiles = (int)rem;
  pl.sk_pieces = P;
  pl.sk_kb = kbs;
  const int64_t g = T < cus ? rem * P : cus;
  pl.grid = (int)g;
}

// Estimated time (us) of a skinny plan with bm x 4wn tiles and a K split of
// s, for 256 < M <= 2048, from the bytes each CU pulls: a workgroup streams
// (bm + 4 wn) rows of its K range; 64 x 64 tiles run two workgroups per CU
// (sharing the CU's rate), the larger ones one; the grid is padded to whole
// groups of 8 units per row tile and runs in rounds of cus (x2) workgroups;
// a split adds its partial store and the last split's read-back.  The
// constants (per-CU rate 60 GB/s with two workgroups, 50 GB/s with one,
// 3.5 us launch, 3 us fix-up latency) were tuned on forced-plan timings of
// 40 shapes at 288-512 rows: the plan they pick was on average 1% and at
// most 16% slower than the fastest plan timed for the shape.
double skinny_cost_us(int64_t M, int64_t N, int64_t K, int bm, int wn, int s, int cus) {
  const int64_t KB = K / 128;
  const int64_t kbs = ceil_div(KB, s);
  s = (int)ceil_div(KB, kbs);
  const int64_t bn = 4 * wn;
  const int64_t mt = ceil_div(M, bm), nt = ceil_div(N, bn);
  const int occ = (bm == 64 && wn == 16) ? 2 : 1;
  const int64_t grid = ceil_div(nt * s, 8) * 8 * mt;
  const double bytes = (double)((bm + bn) * kbs * 128);
  const double rounds = (double)ceil_div(grid, (int64_t)cus * occ);
  double t = (occ == 2 && grid > cus) ? rounds * 2.0 * bytes / 60e3 : rounds * bytes / 50e3;
  if (s > 1) t += 3.0 + (double)s * (double)(bm * bn * 4) / 50e3;
  return 3.5 + t;
}

// The skinny plan of least estimated time over 64 x 64, 64 x 128 and
// 128 x 128 tiles and K splits of 1-4; a split only where its workgroups
// still run in one round (so its partials stay within 16 MiB) and fit the
// workspace.  Returns the estimate.
double best_skinny(int64_t M, int64_t N, int64_t K, int cus, size_t ws_bytes, int* bm, int* wn, int* splits) {
  const int shapes[3][2] = {{64, 16}, {64, 32}, {128, 32}};
  double best = -1.0;
  for (const auto& sh : shapes) {
    const int64_t mt = ceil_div(M, sh[0]), nt = ceil_div(N, 4 * sh[1]);
    const int occ = sh[0] == 64 && sh[1] == 16 ? 2 : 1;
    const int cap = (int)(K / (20 * sh[0]));
    for (int s = 1; s <= 4; ++s) {
      if (s > 1 && (s > cap || mt * nt * s > (int64_t)cus * occ || mt * nt > dg::kWsMaxCounters ||
                    dg::skinny_workspace_bytes(sh[0], (int)mt, (int)nt, sh[1], s) > ws_bytes))
        break;
      const double t = skinny_cost_us(M, N, K, sh[0], sh[1], s, cus);
      if (best < 0.0 || t < best) {
        best = t;
        *bm = sh[0];
        *wn = sh[1];
        *splits = s;
      }
    }
  }
  return best;
}

// Estimated time (us) of a 256 x 128 tile plan: its whole rounds of tiles,
// then the tail's K pieces and their fix-up (the last piece of a tile reads
// the others' 128 KB partials).  Constants fitted to default-plan timings of
// 126 shapes at 129-2048 rows (per-CU rate 61 GB/s, 9.5 us fixed, 5.5 us
// fix-up latency; mean error 10%).
double persistent_cost_us(const DensePlan& pl, int64_t K) {
  const double tb = 384.0 * 128.0;  // A and B bytes of one K block of a tile
  double t = pl.dp_tiles ? (double)ceil_div(pl.dp_tiles, pl.grid) * (double)(K / 128) * tb / 61e3 : 0.0;
  if (pl.sk_tiles) {
    t += (double)pl.sk_kb * tb / 61e3;
    if (pl.sk_pieces > 1) t += 5.5 + (double)pl.sk_pieces * 256.0 * 128.0 * 4.0 / 61e3;
  }
  return 9.5 + t;
}

// Skinny kernel (one workgroup per CU): column width and K split chosen so
// the workgroups fill the CUs in whole rounds.  Without a split the wider
// tile wins ties; with one, 16-column waves give the most tiles, and the split
// is at most K / (20 bm) (the fp32 partials then stay below a fifth of the
// weight bytes; more splits lose more in the fix-up than they gain), at most
// 16, and only as large as the workspace holds.  (Re-measured against a sweep
// of tile shape, split and ring depth on the decode shapes of the dense sweep,
// each configuration with a freshly zeroed workspace: no configuration beat
// this rule by more than the run-to-run spread.)
void plan_skinny(DensePlan& pl, int64_t M, int64_t N, int64_t K, int cus, size_t ws_bytes) {
  const int KB = (int)(K / 128);
  pl.skinny = true;
  // 64 < M <= 128: one 128-row tile (weights read once) when the columns
  // alone nearly fill the CUs; otherwise two 64-row tiles, whose split-K
  // partials are half as large per tile.  128 < M <= 256: 64-row tiles of 64
  // columns (measured fastest there against 128 x 128 tiles)
  pl.cfg = (M <= 64 || M > 128 || ceil_div(N, 64) < cus / 2) ? 64 : 128;
  pl.m_tiles = (int)ceil_div(M, pl.cfg);
  const int64_t t16 = pl.m_tiles * ceil_div(N, 64);
  const int64_t t32 = pl.m_tiles * ceil_div(N, 128);
  auto fill = [&](int64_t t) { return (double)t / (double)(ceil_div(t, cus) * cus); };
  pl.wn = (M <= 128 && t16 >= cus && fill(t32) >= fill(t16)) ? 32 : 16;
  int cap_rows = pl.cfg;  // K split capped at K / (20 * cap_rows): partials (splits * bm * 4 B per column) <= K / 5
  // 64 < M <= 128 with two 64-row tiles: each streams all of A beside its
  // columns of B; one 128 x 128 tile halves those A reads, and wins where it
  // still fills the CUs through a K split (partials then up to K / 2.5 per column)
  if (M > 64 && M <= 128 && pl.cfg == 64) {
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
  if (tiles < cus && tiles <= dg::kWsMaxCounters) {
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
  if (M > 256) {  // 256 < M <= 2048: the tile shape and split of least estimated time
    best_skinny(M, N, K, cus, ws_bytes, &pl.cfg, &pl.wn, &splits);
    pl.m_tiles = (int)ceil_div(M, pl.cfg);
    pl.n_tiles = (int)ceil_div(N, 4 * pl.wn);
  }
  int depth = dg::skinny_depth(pl.cfg, pl.wn);
  const Force f = forced();
  if (f.sk_bm) {  // DG_FORCE_CONFIG=skinny=...
    pl.cfg = f.sk_bm;
    pl.wn = f.sk_wn;
    pl.m_tiles = (int)ceil_div(M, pl.cfg);
    pl.n_tiles = (int)ceil_div(N, 4 * pl.wn);
    splits = f.sk_splits < KB ? f.sk_splits : KB;
    if ((int64_t)pl.m_tiles * pl.n_tiles > dg::kWsMaxCounters) splits = 1;
    while (splits > 1 && dg::skinny_workspace_bytes(pl.cfg, pl.m_tiles, pl.n_tiles, pl.wn, splits) > ws_bytes) --splits;
    depth = f.sk_depth;
  }
  pl.depth = depth;
  // whole ring cycles per split where that does not cost a split
  int kbs = (int)ceil_div(KB, splits);
  const int kbs_r = (int)ceil_div(kbs, depth) * depth;
  if (ceil_div(KB, kbs_r) == splits || kbs_r - kbs < depth / 2) kbs = kbs_r;
  pl.kb_per_split = kbs;
  pl.splits = (int)ceil_div(KB, pl.kb_per_split);
}

// The dense forms.  kFp8 / kAcc / kUe8m0: skinny for M <= 128 (for M <= 512
// where 2 ceil(N / 128) <= CUs and K <= 8192, and for M <= 2048 where its
// estimated time beats the 256 x 128 plan's), else 256 x 256 tiles where they fill whole rounds, else
// 256 x 128 tiles with a K-split tail.  kBf16: 256 x 256 tiles where they fill whole rounds, else 256 x 128
// tiles.  DG_FORCE_CONFIG=kernel=... overrides the wide / 256 x 128 choice
// for M > 128 (and for the BF16 form at any M >= 1).
enum DenseKind { kFp8 = 0, kAcc = 1, kUe8m0 = 2, kBf16 = 3 };

DensePlan plan_dense(DenseKind kind, int64_t M, int64_t N, int64_t K, int cus, size_t ws_bytes) {
  DensePlan pl;
  const int64_t kbytes = kind == kBf16 ? 2 * K : K;  // bytes per operand row
  const Force f = forced();
  // 128 < M <= 512: the decode kernel where the output has few columns
  // (2 ceil(N / 128) <= CUs: at most half the CUs' worth of 256 x 128 tiles
  // per row tile, all of them split along K below 257 rows) and K is
  // moderate; measured 1.1-3.4x faster there, and slower at K = 16384 or
  // with more columns
  const bool mid = M > 128 && f.kernel == kForceNone &&
                   ((f.sk_bm && M <= 2048) || (M <= 512 && 2 * ceil_div(N, 128) <= cus && K <= 8192));
  if (kind != kBf16 && (M <= 128 || mid)) {
    plan_skinny(pl, M, N, K, cus, ws_bytes);
    return pl;
  }
  const bool wide =
      f.kernel == kForceWide ? true : f.kernel == kForcePersistent ? false : wide_fill(M, N, cus, kind != kBf16);
  if (wide)
    plan_wide(pl, M, N, kbytes, cus);
  else
    plan_persistent(pl, M, N, kbytes, cus, ws_bytes);
  // 512 < M <= 2048, K <= 8192, on at least 128 CUs (the estimates were
  // fitted on the whole chip): the skinny kernel where its estimate beats the
  // 256 x 128 plan's by 15% (few tiles and short K, where that plan's K-split
  // fix-up dominates: measured up to 3.3x faster; with more tiles or longer K
  // the tile kernel stays)
  if (kind != kBf16 && !wide && f.kernel == kForceNone && M > 512 && M <= 2048 && K <= 8192 && cus >= 128) {
    int bm = 0, wn = 0, s = 0;
    if (1.15 * best_skinny(M, N, K, cus, ws_bytes, &bm, &wn, &s) < persistent_cost_us(pl, K)) {
      pl = DensePlan();
      plan_skinny(pl, M, N, K, cus, ws_bytes);
    }
  }
  return pl;
}

const char* kind_name(DenseKind k) {
  return k == kFp8 ? "gemm_nt" : k == kAcc ? "gemm_nt_acc" : k == kUe8m0 ? "gemm_nt_ue8m0" : "bf16_gemm_nt";
}

// Validation shared by the dense forms past their pointer checks, then one
// launch per row chunk.
int run_dense(DenseKind kind, const uint8_t* A, const void* sfa, const uint8_t* B, const void* sfb, const float* C,
              void* D, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  const int64_t kbytes = kind == kBf16 ? 2 * K : K;
  const int64_t out_bytes = (kind == kAcc ? 4 : 2) * N;
  int rc = check_weights_and_scales(N, kbytes, kind == kBf16 ? 0 : M, kind == kUe8m0 ? ceil_div(K / 128, 4) : K / 128);
  if (rc) return rc;
  const int64_t chunk = launch_rows(kbytes, out_bytes);
  if (chunk == 0) return fail(DG_ERR_SHAPE, "rows of %lld bytes do not fit 32-bit offsets", (long long)kbytes);
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  const int ecus = effective_cus(cus);
  const size_t ws = workspace ? workspace_bytes : 0;
  for (int64_t r0 = 0; r0 < M; r0 += chunk) {
    const int64_t rows = std::min(chunk, M - r0);
    const DensePlan pl = plan_dense(kind, rows, N, K, ecus, ws);
    dg::GemmParams p{};
    p.A = A + r0 * kbytes;
    p.sfa = kind == kBf16 ? nullptr : static_cast<const float*>(sfa) + r0;  // [K/128][M]: a chunk starts r0 floats in
    p.sfa_ld = (int)M;
    p.B = B;
    p.sfb = static_cast<const float*>(sfb);
    if (kind == kAcc) {
      p.Cacc = C ? C + r0 * N : nullptr;
      p.Dacc = static_cast<float*>(D) + r0 * N;
    } else {
      p.D = static_cast<uint16_t*>(D) + r0 * N;
    }
    p.ws = static_cast<float*>(workspace);
    p.index = nullptr;
    p.rows = rows;
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
    if (print_configs()) {
      if (pl.skinny)
        std::fprintf(stderr,
                     "[dg] %s M=%lld N=%lld K=%lld rows=%lld+%lld kernel=skinny tile=%dx%d m_tiles=%d n_tiles=%d splits=%d "
                     "depth=%d weights=%s\n",
                     kind_name(kind), (long long)M, (long long)N, (long long)K, (long long)r0, (long long)rows, pl.cfg,
                     4 * pl.wn, pl.m_tiles, pl.n_tiles, pl.splits, pl.depth,
                     pl.cfg == 64 && pl.m_tiles == 1 ? "nt" : "default");
      else
        std::fprintf(stderr,
                     "[dg] %s M=%lld N=%lld K=%lld rows=%lld+%lld kernel=%s grid=%d tiles=%d whole=%d tail=%d x %d pieces of %d\n",
                     kind_name(kind), (long long)M, (long long)N, (long long)K, (long long)r0, (long long)rows,
                     pl.wide ? "wide" : "persistent", pl.grid, pl.m_tiles * pl.n_tiles, pl.dp_tiles, pl.sk_tiles,
                     pl.sk_pieces, pl.sk_kb);
    }
    const int mode = kind == kFp8 ? dg::kDense : kind == kAcc ? dg::kDenseAcc : kind == kUe8m0 ? dg::kDenseUe8m0
                                                                                                 : dg::kDenseBf16;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = pl.skinny ? dg::launch_gemm_skinny(pl.cfg, pl.wn, pl.depth, kind == kUe8m0, p, st)
                         : pl.wide ? dg::launch_gemm_wide(mode, pl.grid, p, st)
                                   : dg::launch_gemm_persistent(mode, pl.grid, p, st);
    if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

int check_rows(int64_t M, const char* name) {
  if (M < 0) return fail(DG_ERR_SHAPE, "%s must be >= 0 (got %lld)", name, (long long)M);
  if (M > ((int64_t)1 << 31) - 1) return fail(DG_ERR_SHAPE, "%s too large", name);
  return DG_OK;
}

// Contiguous-form plan for one launch of `rows` rows: the wide kernel
// (256 x 256 tiles, passes at expert boundaries) when its tiles fill whole
// rounds of the CUs to >= 85%; else the persistent kernel over 128 x 256
// tiles.  Each workgroup lists its tiles in an LDS table of
// 64 entries, so the grid grows past the CU count when a launch has more
// than 64 tiles per CU.
struct ContigPlan {
  bool wide = false;
  int grid = 0;
  int64_t tiles = 0;
};
ContigPlan plan_contiguous(int64_t rows, int64_t N, int64_t K, int cus) {
  ContigPlan cp;
  const Force f = forced();
  const int64_t tw = ceil_div(rows, 256) * ceil_div(N, 256);
  const bool wide_ok = rows >= 256 && N >= 256;
  const bool wide = f.kernel == kForceWide ? wide_ok
                    : f.kernel == kForcePersistent
                        ? false
                        // at any K: 256 x 256 tiles measured 1-16% faster than 128 x 256 at
                        // K = 512-3072, with aligned and with ragged expert segments
                        : wide_ok && (double)tw / (double)(ceil_div(tw, cus) * cus) >= 0.85;
  const int64_t tiles = wide ? tw : ceil_div(rows, 128) * ceil_div(N, 256);
  const int64_t maxt = wide ? dg::kWideMaxContigTiles : dg::kPersistentMaxContigTiles;
  const int64_t g = std::max<int64_t>(cus, ceil_div(tiles, maxt));
  cp.wide = wide;
  cp.tiles = tiles;
  cp.grid = (int)std::min(tiles, g);
  return cp;
}

// DG_CHECK_LAYOUT: every aligned 128-row block holds rows of at most one
// expert (indices outside [0, G) are padding and free).  Reads m_indices on
// the host, so it synchronises the stream; a stream under capture is not
// checked.
int check_contiguous_layout(const int32_t* m_indices, int64_t M_total, int64_t G, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DG_ERR_DEVICE, "DG_CHECK_LAYOUT: cannot query the stream");
  }
  if (cap != hipStreamCaptureStatusNone) return DG_OK;
  std::vector<int32_t> idx((size_t)M_total);
  if (hipMemcpyAsync(idx.data(), m_indices, (size_t)M_total * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DG_ERR_DEVICE, "DG_CHECK_LAYOUT: reading m_indices failed");
  }
  for (int64_t b = 0; b < M_total; b += 128) {
    int32_t e = -1;
    for (int64_t r = b; r < std::min(M_total, b + 128); ++r) {
      const int32_t x = idx[(size_t)r];
      if (x < 0 || x >= G) continue;
      if (e >= 0 && x != e)
        return fail(DG_ERR_INVALID_ARG,
                    "DG_CHECK_LAYOUT: rows %lld..%lld hold experts %d and %d (segments must be padded to 128 rows)",
                    (long long)b, (long long)std::min(M_total, b + 128) - 1, e, x);
      e = x;
    }
  }
  return DG_OK;
}

// The M-grouped contiguous form with fp32 (ue = false) or packed UE8M0 scales.
int run_contiguous(bool ue, const uint8_t* A, const void* sfa, const uint8_t* B, const void* sfb, uint16_t* D,
                   const int32_t* m_indices, int64_t M_total, int64_t N, int64_t K, int64_t G, void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if ((rc = check_rows(M_total, "M_total"))) return rc;
  if (G < 1 || G > kMaxGroups) return fail(DG_ERR_SHAPE, "G must be in [1, 1024] (got %lld)", (long long)G);
  if (M_total == 0) return ok();
  if ((rc = check_operands(A, sfa, B, sfb, D))) return rc;
  if (!m_indices) return fail(DG_ERR_INVALID_ARG, "null m_indices");
  if (!aligned(m_indices, 4)) return fail(DG_ERR_ALIGN, "m_indices must be 4-byte aligned");
  const int64_t srow = ue ? ceil_div(K / 128, 4) : K / 128;  // scale words per row
  if ((rc = check_weights_and_scales(N, K, M_total, srow))) return rc;
  // row chunks are multiples of 256 rows, so every aligned 128-row block
  // stays inside one chunk
  const int64_t chunk = launch_rows(K, 2 * N);
  if (chunk == 0) return fail(DG_ERR_SHAPE, "rows do not fit 32-bit offsets");
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  if (std::getenv("DG_CHECK_LAYOUT") && (rc = check_contiguous_layout(m_indices, M_total, G, stream))) return rc;
  const int ecus = effective_cus(cus);
  for (int64_t r0 = 0; r0 < M_total; r0 += chunk) {
    const int64_t rows = std::min(chunk, M_total - r0);
    const ContigPlan cp = plan_contiguous(rows, N, K, ecus);
    dg::GemmParams p{};
    p.A = A + r0 * K;
    p.sfa = static_cast<const float*>(sfa) + r0;  // [K/128 or ceil(K/512)][M_total]: a chunk starts r0 words in
    p.sfa_ld = (int)M_total;
    p.B = B;
    p.sfb = static_cast<const float*>(sfb);
    p.D = D + r0 * N;
    p.index = m_indices + r0;
    p.rows = rows;
    p.N = (int)N;
    p.K = (int)K;
    p.G = (int)G;
    p.m_tiles = (int)ceil_div(rows, cp.wide ? 256 : 128);
    p.n_tiles = (int)ceil_div(N, 256);
    p.splits = 1;
    p.kb_per_split = (int)(K / 128);
    p.dp_tiles = (int)cp.tiles;  // every tile whole: no K-split tail, no workspace
    p.sk_tiles = 0;
    p.sk_pieces = 1;
    p.sk_kb = (int)(K / 128);
    if (print_configs())
      std::fprintf(stderr,
                   "[dg] contiguous%s M_total=%lld N=%lld K=%lld G=%lld rows=%lld+%lld tile=%dx256 kernel=%s grid=%d\n",
                   ue ? "_ue8m0" : "", (long long)M_total, (long long)N, (long long)K, (long long)G, (long long)r0,
                   (long long)rows, cp.wide ? 256 : 128, cp.wide ? "wide" : "persistent", cp.grid);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int mode = ue ? dg::kContiguousUe8m0 : dg::kContiguous;
    const hipError_t e =
        cp.wide ? dg::launch_gemm_wide(mode, cp.grid, p, st) : dg::launch_gemm_persistent(mode, cp.grid, p, st);
    if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

// The M-grouped masked form with fp32 (ue = false) or packed UE8M0 scales.
int run_masked(bool ue, const uint8_t* A, const void* sfa, const uint8_t* B, const void* sfb, uint16_t* D,
               const int32_t* masked_m, int64_t G, int64_t max_m, int64_t N, int64_t K, void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (G < 1 || G > kMaxGroups) return fail(DG_ERR_SHAPE, "G must be in [1, 1024] (got %lld)", (long long)G);
  if (max_m < 0) return fail(DG_ERR_SHAPE, "max_m must be >= 0");
  if (max_m > ((int64_t)1 << 31) - 1) return fail(DG_ERR_SHAPE, "max_m too large");
  if (max_m == 0) return ok();
  if ((rc = check_operands(A, sfa, B, sfb, D))) return rc;
  if (!masked_m) return fail(DG_ERR_INVALID_ARG, "null masked_m");
  if (!aligned(masked_m, 4)) return fail(DG_ERR_ALIGN, "masked_m must be 4-byte aligned");
  // each expert's A, alpha, B and D are addressed from the expert's own base
  if ((rc = check_weights_and_scales(N, K, max_m, ue ? ceil_div(K / 128, 4) : K / 128))) return rc;
  if ((max_m + 256) * K >= kOffLim || max_m * N * 2 >= kOffLim)
    return fail(DG_ERR_SHAPE, "one expert's rows exceed 32-bit offsets (max_m = %lld)", (long long)max_m);
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  dg::GemmParams p{};
  p.A = A;
  p.sfa = static_cast<const float*>(sfa);
  p.sfa_ld = (int)max_m;
  p.B = B;
  p.sfb = static_cast<const float*>(sfb);
  p.D = D;
  p.index = masked_m;
  p.rows = max_m;
  p.N = (int)N;
  p.K = (int)K;
  p.G = (int)G;
  // 128 x 256 tiles over a device-side task list
  p.m_tiles = (int)ceil_div(max_m, 128);
  p.n_tiles = (int)ceil_div(N, 256);
  p.splits = 1;
  p.kb_per_split = (int)(K / 128);
  const int64_t tiles = G * p.m_tiles * p.n_tiles;
  const int ecus = effective_cus(cus);
  const int grid = (int)(tiles < ecus ? tiles : ecus);
  if (print_configs())
    std::fprintf(stderr, "[dg] masked%s G=%lld max_m=%lld N=%lld K=%lld tile=128x256 kernel=persistent grid=%d weights=%s\n",
                 ue ? "_ue8m0" : "", (long long)G, (long long)max_m, (long long)N, (long long)K, grid,
                 p.m_tiles == 1 ? "nt" : "default");
  const hipError_t e = dg::launch_gemm_persistent(ue ? dg::kMaskedUe8m0 : dg::kMasked, grid, p,
                                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int dg_fp8_gemm_nt(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb, uint16_t* D, int64_t M,
                   int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if ((rc = check_rows(M, "M"))) return rc;
  if (M == 0) return ok();
  if ((rc = check_operands(A, sfa, B, sfb, D))) return rc;
  if ((rc = check_workspace(workspace, workspace_bytes))) return rc;
  return run_dense(kFp8, A, sfa, B, sfb, nullptr, D, M, N, K, workspace, workspace_bytes, stream);
}

int dg_fp8_gemm_nt_noalloc(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb, uint16_t* D,
                           int64_t M, int64_t N, int64_t K, void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if ((rc = check_rows(M, "M"))) return rc;
  if (M == 0) return ok();
  if ((rc = check_operands(A, sfa, B, sfb, D))) return rc;
  if ((rc = check_weights_and_scales(N, K, M, K / 128))) return rc;
  const int64_t chunk = launch_rows(K, 2 * N);
  if (chunk == 0) return fail(DG_ERR_SHAPE, "rows of %lld bytes do not fit 32-bit offsets", (long long)K);
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  // the plan dg_fp8_gemm_nt makes with a full workspace; every row chunk's
  // split-K scratch must fit the static array
  const int ecus = effective_cus(cus);
  for (int64_t r0 = 0; r0 < M; r0 += chunk) {
    const DensePlan pl = plan_dense(kFp8, std::min(chunk, M - r0), N, K, ecus, (size_t)-1);
    const size_t need = pl.skinny ? dg::skinny_workspace_bytes(pl.cfg, pl.m_tiles, pl.n_tiles, pl.wn, pl.splits)
                        : (pl.persist && !pl.wide) ? dg::persistent_workspace_bytes(pl.sk_tiles, pl.sk_pieces)
                                                   : 0;
    if (need > dg::kScratchBytes)
      return fail(DG_ERR_WORKSPACE,
                  "this shape's split-K scratch (%zu bytes) exceeds the static maximum of %zu bytes; "
                  "use dg_fp8_gemm_nt with a workspace",
                  need, dg::kScratchBytes);
  }
  void* scratch = nullptr;
  const hipError_t e = dg::scratch_for_current_device(&scratch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "static scratch unavailable: %s", hipGetErrorString(e));
  return run_dense(kFp8, A, sfa, B, sfb, nullptr, D, M, N, K, scratch, dg::kScratchBytes, stream);
}

int dg_fp8_gemm_nt_acc(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb, const float* C,
                       float* D, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if ((rc = check_rows(M, "M"))) return rc;
  if (M == 0) return ok();
  if ((rc = check_operands(A, sfa, B, sfb, D))) return rc;
  if (C && !aligned(C, 16)) return fail(DG_ERR_ALIGN, "A, B, C and D must be 16-byte aligned");
  if ((rc = check_workspace(workspace, workspace_bytes))) return rc;
  return run_dense(kAcc, A, sfa, B, sfb, C, D, M, N, K, workspace, workspace_bytes, stream);
}

int dg_fp8_gemm_nt_ue8m0(const uint8_t* A, const int32_t* sfa, const uint8_t* B, const int32_t* sfb, uint16_t* D,
                         int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if ((rc = check_rows(M, "M"))) return rc;
  if (M == 0) return ok();
  if ((rc = check_operands(A, sfa, B, sfb, D))) return rc;
  if ((rc = check_workspace(workspace, workspace_bytes))) return rc;
  return run_dense(kUe8m0, A, sfa, B, sfb, nullptr, D, M, N, K, workspace, workspace_bytes, stream);
}

int dg_bf16_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* D, int64_t M, int64_t N, int64_t K,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (K <= 0 || K % 64 != 0) return fail(DG_ERR_SHAPE, "K must be a positive multiple of 64 (got %lld)", (long long)K);
  if (N <= 0 || N % 16 != 0) return fail(DG_ERR_SHAPE, "N must be a positive multiple of 16 (got %lld)", (long long)N);
  if (K > (int64_t)1 << 29 || N > (int64_t)1 << 30) return fail(DG_ERR_SHAPE, "N or K too large");
  int rc = check_rows(M, "M");
  if (rc) return rc;
  if (M == 0) return ok();
  if (!A || !B || !D) return fail(DG_ERR_INVALID_ARG, "null operand pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16))
    return fail(DG_ERR_ALIGN, "A, B and D must be 16-byte aligned");
  if ((rc = check_workspace(workspace, workspace_bytes))) return rc;
  return run_dense(kBf16, reinterpret_cast<const uint8_t*>(A), nullptr, reinterpret_cast<const uint8_t*>(B), nullptr,
                   nullptr, D, M, N, K, workspace, workspace_bytes, stream);
}

int dg_k_grouped_fp8_gemm_nt_contiguous(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb,
                                        const float* C, float* D, const int32_t* ks, int64_t G, int64_t M,
                                        int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (G < 1 || G > kMaxGroups) return fail(DG_ERR_SHAPE, "G must be in [1, 1024] (got %lld)", (long long)G);
  if ((rc = check_rows(M, "M"))) return rc;
  if (M == 0) return ok();
  if (!A || !sfa || !B || !sfb || !D || !ks) return fail(DG_ERR_INVALID_ARG, "null operand pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || (C && !aligned(C, 16)))
    return fail(DG_ERR_ALIGN, "A, B, C and D must be 16-byte aligned");
  if (!aligned(sfa, 4) || !aligned(sfb, 4) || !aligned(ks, 4))
    return fail(DG_ERR_ALIGN, "scale arrays and ks must be 4-byte aligned");
  // one tile grid per group over the shared operands, addressed with 32-bit
  // offsets; fp32 C and D are addressed per group
  if ((M + 256) * K >= kOffLim || (N + 256) * K >= kOffLim || (M + 256) * N * 4 >= kOffLim ||
      std::max(M, N) * (K / 128) * 4 >= kOffLim)
    return fail(DG_ERR_SHAPE, "problem too large for 32-bit buffer offsets");
  int cus = 0;
  if ((rc = check_device(&cus))) return rc;
  dg::GemmParams p{};
  p.A = A;
  p.sfa = sfa;
  p.sfa_ld = (int)M;
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
  const Force f = forced();
  const bool wide = f.kernel == kForceWide         ? (M >= 256 && N >= 256)
                    : f.kernel == kForcePersistent ? false
                                                   : kgrouped_wide(G, M, N, ecus);
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
  if (print_configs())
    std::fprintf(stderr, "[dg] k_grouped G=%lld M=%lld N=%lld K=%lld kernel=%s tiles=%lld grid=%d\n", (long long)G,
                 (long long)M, (long long)N, (long long)K, wide ? "wide" : "persistent", (long long)tiles, grid);
  const hipError_t e = wide ? dg::launch_gemm_wide(dg::kKGrouped, grid, p, static_cast<hipStream_t>(stream))
                            : dg::launch_gemm_persistent(dg::kKGrouped, grid, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}


int dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb,
                                        uint16_t* D, const int32_t* m_indices, int64_t M_total, int64_t N,
                                        int64_t K, int64_t G, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return run_contiguous(false, A, sfa, B, sfb, D, m_indices, M_total, N, K, G, stream);
}

int dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const uint8_t* A, const int32_t* sfa, const uint8_t* B,
                                              const int32_t* sfb, uint16_t* D, const int32_t* m_indices,
                                              int64_t M_total, int64_t N, int64_t K, int64_t G, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return run_contiguous(true, A, sfa, B, sfb, D, m_indices, M_total, N, K, G, stream);
}


int dg_m_grouped_fp8_gemm_nt_masked(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb,
                                    uint16_t* D, const int32_t* masked_m, int64_t G, int64_t max_m, int64_t N,
                                    int64_t K, int64_t expected_m, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  (void)expected_m;  // launch shape and results never depend on it
  return run_masked(false, A, sfa, B, sfb, D, masked_m, G, max_m, N, K, stream);
}

int dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const uint8_t* A, const int32_t* sfa, const uint8_t* B, const int32_t* sfb,
                                          uint16_t* D, const int32_t* masked_m, int64_t G, int64_t max_m, int64_t N,
                                          int64_t K, int64_t expected_m, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  (void)expected_m;
  return run_masked(true, A, sfa, B, sfb, D, masked_m, G, max_m, N, K, stream);
}

int dg_quant_1x128(const float* x, uint8_t* q, float* sfa, int64_t G, int64_t M, int64_t K, void* stream) {
  if (K <= 0 || K % 128) return fail(DG_ERR_SHAPE, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  if (G < 0 || M < 0) return fail(DG_ERR_SHAPE, "G and M must be >= 0");
  // grid (ceil(M / 16) * (K / 128), G)
  if (G > 65535 || M > ((int64_t)1 << 31) - 16 || ceil_div(M, 16) * (K / 128) > ((int64_t)1 << 31) - 1)
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
  // grid (ceil(M / 16) * (K / 128), G)
  if (G > 65535 || M > ((int64_t)1 << 31) - 16 || ceil_div(M, 16) * (K / 128) > ((int64_t)1 << 31) - 1)
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
  const int ecus = effective_cus(query_cus());
  const int64_t kbytes = op == DG_OP_BF16_GEMM_NT ? 2 * K : K;
  // the largest row chunk's plan; chunks reuse the workspace one after another
  const int64_t chunk = launch_rows(kbytes, 2 * N);
  if (chunk == 0) return 0;
  const int64_t r = std::min(rows, chunk);
  const DenseKind kind = op == DG_OP_BF16_GEMM_NT ? kBf16 : op == DG_OP_GEMM_NT_UE8M0 ? kUe8m0 : kFp8;
  size_t need = 0;
  // the fp8 forms: the accumulating one shares this workspace and plans the same
  // way, except that it has 256 x 128 tiles where the bf16-output form has 256 x 256
  const DenseKind kinds[2] = {kind, kAcc};
  for (int i = 0; i < (kind == kFp8 ? 2 : 1); ++i) {
    const DensePlan pl = plan_dense(kinds[i], r, N, K, ecus, (size_t)-1);
    size_t b = 0;
    if (pl.skinny && pl.splits > 1) b = dg::skinny_workspace_bytes(pl.cfg, pl.m_tiles, pl.n_tiles, pl.wn, pl.splits);
    if (pl.persist && !pl.wide) b = dg::persistent_workspace_bytes(pl.sk_tiles, pl.sk_pieces);
    need = std::max(need, b);
  }
  return (need + 15) / 16 * 16;
}

const char* dg_describe_plan(int op, int64_t rows, int64_t N, int64_t K, int64_t G) {
  thread_local std::string text;
  text.clear();
  if ((op != DG_OP_GEMM_NT && op != DG_OP_CONTIGUOUS && op != DG_OP_GEMM_NT_UE8M0 && op != DG_OP_BF16_GEMM_NT &&
       op != DG_OP_K_GROUPED && op != DG_OP_MASKED) ||
      rows <= 0 || N <= 0 || K <= 0 || K % (op == DG_OP_BF16_GEMM_NT ? 64 : 128) || N % 16)
    return text.c_str();
  const int ecus = effective_cus(query_cus());
  char buf[320];
  if (op == DG_OP_CONTIGUOUS) {
    const int64_t chunk = launch_rows(K, 2 * N);
    if (chunk == 0) return text.c_str();
    const int64_t r = std::min(rows, chunk);
    const ContigPlan cp = plan_contiguous(r, N, K, ecus);
    std::snprintf(buf, sizeof(buf), "kernel=%s tile=%dx256 grid=%d tiles=%lld chunks=%lld", cp.wide ? "wide" : "persistent",
                  cp.wide ? 256 : 128, cp.grid, (long long)cp.tiles, (long long)ceil_div(rows, chunk));
    text = buf;
    return text.c_str();
  }
  if (op == DG_OP_MASKED) {  // rows = max_m, G experts; the weights stream non-temporally with one row tile
    const int64_t g = G < 1 ? 1 : G;
    const int64_t mt = ceil_div(rows, 128);
    const int64_t tiles = g * mt * ceil_div(N, 256);
    std::snprintf(buf, sizeof(buf), "kernel=persistent tile=128x256 grid=%lld max_tiles=%lld weights=%s",
                  (long long)(tiles < ecus ? tiles : ecus), (long long)tiles, mt == 1 ? "nt" : "default");
    text = buf;
    return text.c_str();
  }
  if (op == DG_OP_K_GROUPED) {
    const int64_t g = G < 1 ? 1 : G;
    const Force f = forced();
    const bool wide = f.kernel == kForceWide         ? (rows >= 256 && N >= 256)
                      : f.kernel == kForcePersistent ? false
                                                     : kgrouped_wide(g, rows, N, ecus);
    const int64_t tiles = g * ceil_div(rows, 256) * ceil_div(N, wide ? 256 : 128);
    std::snprintf(buf, sizeof(buf), "kernel=%s tile=256x%d grid=%lld tiles=%lld", wide ? "wide" : "persistent",
                  wide ? 256 : 128, (long long)(tiles < ecus ? tiles : ecus), (long long)tiles);
    text = buf;
    return text.c_str();
  }
  const DenseKind kind = op == DG_OP_BF16_GEMM_NT ? kBf16 : op == DG_OP_GEMM_NT_UE8M0 ? kUe8m0 : kFp8;
  const int64_t kbytes = kind == kBf16 ? 2 * K : K;
  const int64_t chunk = launch_rows(kbytes, 2 * N);
  if (chunk == 0 || (N + 256) * kbytes >= kOffLim) return text.c_str();
  const int64_t r = std::min(rows, chunk);
  const DensePlan pl = plan_dense(kind, r, N, K, ecus, (size_t)-1);
  if (pl.skinny)
    std::snprintf(buf, sizeof(buf), "kernel=skinny tile=%dx%d tiles=%d splits=%d weights=%s chunks=%lld", pl.cfg,
                  4 * pl.wn, pl.m_tiles * pl.n_tiles, pl.splits, pl.cfg == 64 && pl.m_tiles == 1 ? "nt" : "default",
                  (long long)ceil_div(rows, chunk));
  else
    std::snprintf(buf, sizeof(buf), "kernel=%s tile=%dx%d grid=%d tiles=%d whole=%d tail=%dx%d chunks=%lld",
                  pl.wide ? "wide" : "persistent", 256, pl.wide ? 256 : 128, pl.grid, pl.m_tiles * pl.n_tiles,
                  pl.dp_tiles, pl.sk_tiles, pl.sk_pieces, (long long)ceil_div(rows, chunk));
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

const char* dg_version(void) { return "dg-mi355x 0.2.0 (gfx950)"; }

}  // extern "C"
