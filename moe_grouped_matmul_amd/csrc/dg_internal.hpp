// Internal declarations shared by the host layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Parameters of one GEMM launch (dense, contiguous or masked form).
struct GemmParams {
  const uint8_t* A;      // e4m3 activations
  const float* sfa;      // activation scales, MN-major [K/128][rows] (per group when masked)
  const uint8_t* B;      // e4m3 weights [G][N][K]
  const float* sfb;      // weight scales [G][ceil(N/128)][K/128]
  uint16_t* D;           // bf16 output
  const float* Cacc;     // accumulating forms: fp32 C [G][rows][N] (null: zero), fp32 D below
  float* Dacc;           // accumulating forms: fp32 output D = C + A . B^T (may equal Cacc)
  float* ws;             // split-K partials [splits][rows][N] (dense only)
  const int32_t* index;  // m_indices (contiguous), masked_m (masked) or ks (K-grouped); unused when dense
  int64_t rows;          // dense: M; contiguous: M_total; masked: max_m (rows per group)
  int sfa_ld;            // row stride of the MN-major activation scales (elements): the caller's row
                         // count, which exceeds `rows` when a call is split into row chunks
  int N;
  int K;
  int G;
  int m_tiles;
  int n_tiles;
  int splits;
  int kb_per_split;
  // persistent kernel (gemm_persist.hip): tiles run whole (tile ids
  // [0, dp_tiles)), and tail tiles [dp_tiles, dp_tiles + sk_tiles) each split
  // into sk_pieces pieces of sk_kb K blocks (dense only)
  int dp_tiles;
  int sk_tiles;
  int sk_pieces;
  int sk_kb;
};

// kDenseBf16: the dense schedule over bf16 operands (no scales): a K block
// is 64 bf16 = 128 bytes per row, the same LDS row as an fp8 K block.
// kDenseAcc: the dense fp8 schedule with the fp32 accumulating epilogue
// (D = C + A . B^T).
// kKGrouped: groups along K (index = ks, the K length of each group), A
// [rows][K] and B [N][K] shared by all groups, per-row 1x128 scales on both
// operands (sfa [K/128][rows], sfb [K/128][N]) and one fp32 output
// D[g] = C[g] + A[:, seg g] . B[:, seg g]^T per group.
// kDenseUe8m0: the dense schedule with UE8M0 scales packed four per int32
// along K (sfa [ceil(KB/4)][rows], sfb [ceil(N/128)][ceil(KB/4)]), applied
// by the matrix cores' block scaling; kContiguousUe8m0 / kMaskedUe8m0: the
// M-grouped forms with those scales (sfb per expert; masked sfa
// [G][ceil(KB/4)][max_m]).
enum GemmMode {
  kDense = 0,
  kContiguous = 1,
  kMasked = 2,
  kDenseBf16 = 3,
  kDenseAcc = 4,
  kKGrouped = 5,
  kDenseUe8m0 = 6,
  kContiguousUe8m0 = 7,
  kMaskedUe8m0 = 8
};

// Split-K workspace layout shared by the skinny and persistent kernels: the
// first kWsCounterBytes hold one uint32 completion counter per split tile
// (at most kWsMaxCounters), the fp32 partials follow.  The counters sit at a
// fixed place, zero on entry and left zero by every launch, so one workspace
// serves any sequence of shapes (partials of one call never land where
// another call keeps its counters).
constexpr int kWsMaxCounters = 1024;
constexpr size_t kWsCounterBytes = 4 * kWsMaxCounters;

// Enqueue the skinny dense kernel (gemm_skinny.hip, M <= 128, bm-row tiles
// with bm in {64, 128}, wn in {16, 32} columns per wave, 4 waves):
// p.m_tiles = ceil(M / bm), p.n_tiles = ceil(N / (4 wn)), p.splits K splits of
// p.kb_per_split blocks.  With p.splits > 1 (then at most kWsMaxCounters
// tiles), p.ws must hold skinny_workspace_bytes(...) bytes laid out as above.
// ue: UE8M0 scales packed four per int32 along K (sfa [ceil(KB/4)][rows],
// sfb [ceil(N/128)][ceil(KB/4)]); p.Dacc selects the fp32 accumulating
// epilogue (fp32 scales only).
size_t skinny_workspace_bytes(int bm, int m_tiles, int n_tiles, int wn, int splits);
hipError_t launch_gemm_skinny(int bm, int wn, int depth, bool ue, const GemmParams& p, hipStream_t stream);
// K blocks in flight per wave (ring depth; LDS per slot is (bm + 4 wn) * 128 B
// plus 1 KB); a split's block count is padded to a multiple of it (padding
// blocks read as zeros), so splits should be multiples.  Four slots for 64-row
// tiles of 16-column waves (about 70 KB, two workgroups per CU) measured
// faster than eight (one per CU) on every decode shape tried.
constexpr int skinny_depth(int bm, int wn) { return bm == 64 ? 4 : (wn == 16 ? 6 : 4); }
// Ring depths compiled for each tile shape (the default above, and deeper
// rings that fit the LDS for measurement through DG_FORCE_CONFIG).
constexpr bool skinny_depth_ok(int bm, int wn, int d) {
  return d == skinny_depth(bm, wn) || (bm == 64 && wn == 16 && d == 8) || (bm == 64 && wn == 32 && d == 6);
}

// Enqueue the persistent kernel (gemm_persist.hip) with `grid` workgroups (one
// per CU): mode kDense over 256x128 tiles (tail tiles split along K when
// p.sk_tiles > 0, at most kWsMaxCounters of them; p.ws then holds
// persistent_workspace_bytes(...) bytes laid out as above), kContiguous over 128x256
// tiles (p.dp_tiles = all tiles, no split; at most kPersistentMaxContigTiles
// tiles per workgroup), kMasked over 128x256 tiles (G <= 1024) or kKGrouped
// over 256x128 tiles of every group (G <= 1024, no split).  One launch's A,
// alpha and D (masked: one group's, from the group's base) and one expert's
// B are addressed with 32-bit offsets; alpha rows are p.sfa_ld apart.
constexpr int kPersistentMaxContigTiles = 64;
size_t persistent_workspace_bytes(int sk_tiles, int sk_pieces);
hipError_t launch_gemm_persistent(int mode, int grid, const GemmParams& p, hipStream_t stream);

// Enqueue the wide-tile persistent kernel (gemm_wide.hip): mode kDense or
// kContiguous over 256 x 256 tiles (p.m_tiles = ceil(rows/256), p.n_tiles =
// ceil(N/256)), no K split, `grid` workgroups; contiguous: at most
// kWideMaxContigTiles tiles per workgroup; offsets as for the persistent
// kernel.
constexpr int kWideMaxContigTiles = 64;
hipError_t launch_gemm_wide(int mode, int grid, const GemmParams& p, hipStream_t stream);

// Static split-K scratch of dg_fp8_gemm_nt_noalloc (noalloc.hip): one array
// of kScratchBytes per device, laid out as a workspace (counters first).
// scratch_for_current_device returns its device address for the current
// device (resolved once per device; the first call also clears the counter
// area with a fill kernel on `stream`).
constexpr size_t kScratchBytes = (size_t)40 << 20;
hipError_t scratch_for_current_device(void** out, hipStream_t stream);

// ue8m0: scales as packed UE8M0 codes (int32 words of four K blocks) instead of fp32
hipError_t launch_quant_1x128(const float* x, uint8_t* q, void* sfa, int64_t G, int64_t M, int64_t K, bool ue8m0,
                              hipStream_t stream);
hipError_t launch_quant_128x128(const float* x, uint8_t* q, void* sfb, int64_t G, int64_t N, int64_t K, bool ue8m0,
                                hipStream_t stream);

}  // namespace dg
