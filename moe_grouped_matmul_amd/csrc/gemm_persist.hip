// Persistent block-scaled FP8 GEMM for gfx950 (and, in mode kDenseBf16, the
// plain BF16 GEMM on the same schedule): one 512-thread workgroup per
// CU walks a list of output tiles (256 x 128; 128 x 256 for the M-grouped
// forms: an aligned 128-row block of the contiguous form belongs to one
// expert, and a masked expert's rows fill fewer padded MFMA rows) with one
// continuous LDS ring, so the next tile's first K blocks load while the
// current tile finishes and stores.  Used for the dense forms with M > 128
// where 256 x 256 tiles (gemm_wide.hip) would leave a partial round, for the
// masked form, and for the contiguous and K-grouped forms where the wide
// kernel does not take them (the contiguous form with K < 4096, or tiles
// leaving a partial round).
//
// The computation is the one of Lesson 13 (hpc.payai.win), Fig. 13-1 and its
// closed-form equation: for every 128-wide K block the fp8 partial product of
// a tile is formed by the matrix cores and promoted into an fp32 accumulator
// with alpha[row, k] * beta[k]; the epilogue rounds to bf16.
//
// Tile scheduler:
//   * dense: tile ids are walked round-robin over the workgroups (id b, b + G,
//     ...), each id mapped so that the 8 XCDs run contiguous, m-grouped tile
//     ranges (operand reuse in each XCD's L2).  When the tile count leaves a
//     partial last round, those tail tiles are split along K into P pieces
//     run by otherwise idle workgroups: each piece stores an fp32 partial tile
//     (coherent across XCDs) and the last piece of a tile to finish (agent-
//     scope counter) sums the partials in piece order and writes bf16, so the
//     result does not depend on the order in which pieces finish;
//   * contiguous (Lesson 13, Fig. 13-3, contiguous layout): the tiles run in
//     lockstep rounds of one tile per workgroup, each XCD a contiguous run of
//     the round, so all XCDs work on the same few experts' weights at a time
//     (they then share them through the Infinity Cache; each XCD walking its
//     own eighth of the tiles keeps up to eight experts' weights in flight);
//     at start every workgroup reduces m_indices over the 128 rows of
//     each of its tiles to the tile's expert (the largest index in [0, G)) and
//     a mask of the rows tagged with it, kept in LDS: B and beta come from
//     that expert, and only the masked rows are stored;
//   * masked (Lesson 13, Fig. 13-3, masked layout): every workgroup reads
//     masked_m on the device and builds the prefix sums of the active tiles
//     per group, sum_g ceil(masked_m[g] / 128) * ceil(N / 256); each round
//     hands every XCD a contiguous run of task ids, ids inside a group walk
//     column tiles with that tile's row tiles adjacent (they share the B tile
//     in one L2), and an id is located by binary search, so only the 128-row
//     tiles holding rows below masked_m are computed, only those rows are
//     loaded and stored, and the launch shape is fixed (graph-capturable);
//   * K-grouped (the weight-gradient family of the deep-dive blog, section 3):
//     every workgroup reads the group lengths ks on the device and builds the
//     first K block of each group; the tiles of all groups are walked in
//     rounds of one tile per workgroup, each round mapped XCD-contiguously,
//     so workgroups share the long and the short groups alike.  A tile runs
//     over its group's K blocks only; a group without K blocks runs one
//     iteration over zero operands, so its tiles still store C.  Both
//     operands carry per-row scales: alpha as in the other forms, beta of the
//     tile's 128 columns through a 6-slot LDS ring of its own.
//
// UE8M0 scales (dense, contiguous and masked): alpha and beta are powers of
// two given by their exponent bytes, four K blocks per 32-bit word.  The matrix cores apply
// them (v_mfma_scale_f32_16x16x128_f8f6f4, every 32-K sub-block of a row
// given the row's byte), which is exact, and also do the promotion: the MFMA
// accumulates into the tile's fp32 accumulator.  Its accumulator input is
// added with one round-to-nearest-even after the products' truncating
// alignment, so this equals a separate fp32 add of the scaled block product,
// bit for bit, without the add (8% faster on the 256x256 kernel).
//
// Main loop (one iteration = one K block of one tile): the three ring slots
// are separate LDS arrays; iteration j's operands sit in slot j % 3.  A wave
// reads all its fragments of iteration j, waits for its own loads of
// iteration j + 1 and for its LDS reads, and after one s_barrier refills slot
// j % 3 with iteration j + 3 -- which may belong to the next tile -- then runs
// the MFMAs and promotions of iteration j.  A finished tile is written with
// buffer stores (lanes outside the tile address past the buffer end) while
// the next tile's blocks are already loading.  Operand layout (128-byte LDS
// rows, 16-byte chunk c of row r at c ^ (r % 8)), fragment order and
// promotion are shared with the wide-tile kernel (gemm_wide.hip).

#include "dg_internal.hpp"
#include "gemm_common.hpp"

namespace dg {
namespace {

constexpr int kRsrcWord3 = 0x00020000;     // raw (untyped) buffer, gfx9 family
constexpr int kCoherent = 16;              // sc1: coherent across the XCDs' L2 caches
constexpr int kStream = 2;                 // nt: weight lines that no other task reads
constexpr uint32_t kOOB = 0xFFFFFF00u;     // an offset past every buffer range used here
constexpr int kMaxMaskedGroups = 1024;     // groups the masked task list supports
constexpr int kMaxContigSegs = kPersistentMaxContigTiles;  // tiles per workgroup the contiguous table holds

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcWord3);
}

// One segment of a workgroup's work: K blocks [kb_lo, kb_hi) of one tile.
struct Seg {
  int mt, nt, grp;   // row tile, column tile, group of A/alpha/D rows (masked)
  int bgrp;          // group of B/beta (masked: grp; contiguous: the tile's expert)
  int row_limit;     // rows of the tile that exist (masked: below masked_m)
  int kb_lo, kb_hi;
  int tail;          // -1: whole tile; else index of a K-split tail tile
  int piece;         // piece of that tail tile
  int zero;          // K-grouped tile of a group without K blocks: one iteration over zeros
};

// HASC (fp32-output modes): C is given and read; without it nothing is loaded.
// NT (masked forms with max_m <= 128, one row tile per expert): every weight
// line is read by exactly one task, and the weight loads carry the
// non-temporal cache policy (where two row tiles of an expert share the
// weights through one L2, the default policy keeps the second read a hit).
template <int MODE, bool HASC, bool NT>
__global__ void __launch_bounds__(512) fp8_gemm_persistent_kernel(GemmParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool BF16 = MODE == kDenseBf16;  // bf16 operands, no scales, no promotion
  constexpr bool ACC = MODE == kDenseAcc;    // fp32 output D = C + A . B^T
  constexpr bool KG = MODE == kKGrouped;     // groups along K, per-column beta, fp32 D[g] = C[g] + ...
  constexpr bool F32OUT = ACC || KG;
  // UE8M0 codes, applied by the matrix cores' block scaling (dense and the M-grouped forms)
  constexpr bool UE = MODE == kDenseUe8m0 || MODE == kContiguousUe8m0 || MODE == kMaskedUe8m0;
  // the schedule: dense, contiguous or masked (the UE8M0 grouped modes take those of their form)
  constexpr int FORM = MODE == kContiguousUe8m0 ? kContiguous : (MODE == kMaskedUe8m0 ? kMasked : MODE);
  // 128-row tiles for the grouped forms: a contiguous 128-row block belongs to
  // one expert, and a masked expert's rows fill fewer padded MFMA rows
  constexpr int WGM = FORM == kContiguous || FORM == kMasked ? 2 : 4;
  constexpr int WGN = FORM == kContiguous || FORM == kMasked ? 4 : 2;
  constexpr int TM = 4;
  constexpr int TN = 4;
  constexpr int BM = WGM * 64;
  constexpr int BN = WGN * 64;
  constexpr int NWAVES = 8;
  constexpr int A_INS = BM / 8 / NWAVES;  // 1 KB (8-row) loads per wave per K block
  constexpr int B_INS = BN / 8 / NWAVES;
  constexpr int L_BLOCK = A_INS + B_INS + (BF16 ? 0 : 1);  // + one alpha load per wave
  constexpr int GM = 4;                       // m-tiles per tile group
  static_assert(2 * L_BLOCK < 64, "vmcnt range");

  // ring slots: A rows [0, BM * 128), B rows [BM * 128, SLOT_S), alpha of
  // the tile's rows [SLOT_S, SLOT_BYTES); one array per slot keeps the
  // compiler's tracking of the buffer-to-LDS loads exact
  constexpr int SLOT_S = (BM + BN) * 128;
  constexpr int SLOT_BYTES = SLOT_S + NWAVES * 64 * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[SLOT_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[SLOT_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[SLOT_BYTES];
  // masked: active tiles before each group; K-grouped: first K block of each group
  __shared__ int pref[FORM == kMasked || KG ? kMaxMaskedGroups + 1 : 1];
  __shared__ int mmv[FORM == kMasked ? kMaxMaskedGroups : 1];       // masked_m clamped to [0, max_m]
  // contiguous: expert of each of this workgroup's tiles (-1: none) and the
  // mask of its rows tagged with that expert
  __shared__ int seg_exp[FORM == kContiguous ? kMaxContigSegs : 1];
  __shared__ uint32_t seg_mask[FORM == kContiguous ? kMaxContigSegs : 1][4];
  __shared__ int last_piece;
  // K-grouped: beta of the tile's BN columns, slot j % 6 for iteration j (the
  // loads of iteration j + 3 go to another slot than the reads of iteration j)
  __shared__ __attribute__((aligned(16))) float bring[KG ? 6 : 1][KG ? BN : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN;
  const int wn = wave % WGN;
  const int q = lane >> 4;
  const int b = (int)blockIdx.x;
  const int G = (int)gridDim.x;

  const int K = BF16 ? 2 * p.K : p.K;  // bytes per operand row
  const int N = p.N;
  const int KB = K >> 7;
  const int KW = (KB + 3) >> 2;  // UE8M0: packed words (four K blocks) per scale row
  const int NB = (N + 127) >> 7;
  const int rows = (int)p.rows;  // dense: M; masked: max_m
  const int ngrp = FORM == kMasked ? p.G : 1;         // groups of A, alpha and D rows
  const int nbgrp = FORM == kContiguous || FORM == kMasked ? p.G : 1;  // groups of B and beta

  // ---- task list
  int T;  // tasks: dense tiles / active masked tiles
  if (FORM == kMasked) {
    if (wave == 0) {
      int carry = 0;
      for (int base = 0; base < ngrp; base += 64) {
        const int g = base + lane;
        int v = 0;
        if (g < ngrp) {
          int mm = p.index[g];
          mm = mm < 0 ? 0 : (mm > rows ? rows : mm);
          mmv[g] = mm;
          v = ((mm + BM - 1) / BM) * p.n_tiles;
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_up(v, off);
          if (lane >= off) v += o;
        }
        if (g < ngrp) pref[g + 1] = carry + v;
        carry += __shfl(v, 63);
      }
      if (lane == 0) pref[0] = 0;
    }
    __syncthreads();
    T = __builtin_amdgcn_readfirstlane(pref[ngrp]);
  } else if constexpr (KG) {
    // pref[g] = first K block of group g: prefix of floor(ks / 128), clamped to KB
    if (wave == 0) {
      int carry = 0;
      for (int base = 0; base < p.G; base += 64) {
        const int g = base + lane;
        int v = 0;
        if (g < p.G) {
          const int k = p.index[g];
          v = k > 0 ? (k >> 7) : 0;
          v = v < KB ? v : KB;
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_up(v, off);
          if (lane >= off) v += o;
        }
        if (g < p.G) pref[g + 1] = carry + v < KB ? carry + v : KB;
        carry += __shfl(v, 63);
        carry = carry < KB ? carry : KB;
      }
      if (lane == 0) pref[0] = 0;
    }
    __syncthreads();
    T = p.G * p.m_tiles * p.n_tiles;
  } else {
    T = p.m_tiles * p.n_tiles;
  }
  const int dp_tiles = FORM == kMasked || KG ? T : p.dp_tiles;  // tasks run as whole tiles
  const int P = p.sk_pieces;                               // pieces per tail tile (dense)
  const int n_dp = b < dp_tiles ? (dp_tiles - b + G - 1) / G : 0;
  const bool has_tail = (MODE == kDense || BF16 || ACC || MODE == kDenseUe8m0) && b < p.sk_tiles * P;
  const int nseg = n_dp + (has_tail ? 1 : 0);
  if (nseg == 0) return;  // uniform over the workgroup

  if constexpr (FORM == kContiguous) {
    // expert and tagged-row mask of each of this workgroup's tiles (the host
    // keeps nseg <= kMaxContigSegs); one wave per tile, two rows per lane
    for (int s = wave; s < nseg; s += NWAVES) {
      int mt, nt;
      grouped_mn(round_tile(b, s, G, dp_tiles), p.m_tiles, p.n_tiles, GM, &mt, &nt);  // as seg_of below
      const int r0 = mt * BM;
      const int lim = rows - r0 < BM ? rows - r0 : BM;
      const int v0 = lane < lim ? p.index[r0 + lane] : -1;
      const int v1 = lane + 64 < lim ? p.index[r0 + 64 + lane] : -1;
      int e = v0 >= 0 && v0 < p.G ? v0 : -1;
      if (v1 >= 0 && v1 < p.G && v1 > e) e = v1;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const int o = __shfl_xor(e, off);
        e = o > e ? o : e;
      }
      const unsigned long long m0 = __ballot(e >= 0 && v0 == e);
      const unsigned long long m1 = __ballot(e >= 0 && v1 == e);
      if (lane == 0) {
        seg_exp[s] = e;
        seg_mask[s][0] = (uint32_t)m0;
        seg_mask[s][1] = (uint32_t)(m0 >> 32);
        seg_mask[s][2] = (uint32_t)m1;
        seg_mask[s][3] = (uint32_t)(m1 >> 32);
      }
    }
    __syncthreads();
  }

  auto seg_of = [&](int s) -> Seg {
    Seg r;
    r.grp = 0;
    r.bgrp = 0;
    r.tail = -1;
    r.piece = 0;
    r.zero = 0;
    r.kb_lo = 0;
    r.kb_hi = KB;
    int d;
    if (s < n_dp) {
      d = b + s * G;
    } else {
      r.tail = b / P;
      r.piece = b - r.tail * P;
      d = dp_tiles + r.tail;
      r.kb_lo = r.piece * p.sk_kb;
      r.kb_hi = r.kb_lo + p.sk_kb < KB ? r.kb_lo + p.sk_kb : KB;
    }
    if (FORM == kMasked) {
      // round s of one task per workgroup, XCD-contiguous inside the round;
      // inside a group the row tiles of one column tile are adjacent tasks,
      // so they run together on one XCD and share that B tile in its L2
      d = round_tile(b, s, G, T);
      int lo = 0, hi = ngrp - 1;  // largest g with pref[g] <= d
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pref[mid] <= d) lo = mid;
        else hi = mid - 1;
      }
      r.grp = __builtin_amdgcn_readfirstlane(lo);
      r.bgrp = r.grp;
      const int local = d - __builtin_amdgcn_readfirstlane(pref[r.grp]);
      const int mm = __builtin_amdgcn_readfirstlane(mmv[r.grp]);
      const int mtg = (mm + BM - 1) / BM;  // >= 1: the group has tasks
      r.nt = local / mtg;
      r.mt = local - r.nt * mtg;
      r.row_limit = mm - r.mt * BM < BM ? mm - r.mt * BM : BM;
    } else if constexpr (KG) {
      // round s of one tile per workgroup, XCD-contiguous inside the round
      const int t = round_tile(b, s, G, T);
      const int tpg = p.m_tiles * p.n_tiles;
      r.grp = t / tpg;
      r.bgrp = 0;
      grouped_mn(t - r.grp * tpg, p.m_tiles, p.n_tiles, GM, &r.mt, &r.nt);
      r.row_limit = rows - r.mt * BM < BM ? rows - r.mt * BM : BM;
      r.kb_lo = __builtin_amdgcn_readfirstlane(pref[r.grp]);
      r.kb_hi = __builtin_amdgcn_readfirstlane(pref[r.grp + 1]);
      if (r.kb_hi == r.kb_lo) {
        r.zero = 1;
        r.kb_hi = r.kb_lo + 1;
      }
    } else {
      // contiguous: lockstep rounds of G consecutive tiles, each XCD a
      // contiguous run inside the round, so all XCDs work on the same few
      // experts' weights at a time; dense: ids b, b + G, ... (then the tail
      // tiles) mapped so that each XCD runs its own contiguous eighth of the
      // tiles (rounds measured 1% slower on 4096x2112x7168)
      grouped_mn(FORM == kContiguous ? round_tile(b, s, G, dp_tiles) : xcd_tile(d, T), p.m_tiles, p.n_tiles, GM,
                 &r.mt, &r.nt);
      r.row_limit = rows - r.mt * BM < BM ? rows - r.mt * BM : BM;
      if (FORM == kContiguous) {
        const int e = __builtin_amdgcn_readfirstlane(seg_exp[s]);
        r.bgrp = e < 0 ? 0 : e;
        if (e < 0) r.row_limit = 0;  // no row tagged with an expert: nothing loaded or stored
      }
    }
    return r;
  };

  // ---- buffer resources: one group's A, alpha and D (masked: from the
  // group's 64-bit base) and one expert's B, each addressed with 32-bit
  // offsets; alpha rows are sfa_ld apart
  (void)nbgrp;
  const uint32_t a_bytes = (uint32_t)rows * (uint32_t)K;
  const uint32_t b_bytes = (uint32_t)N * (uint32_t)K;
  // (the last scale row ends after this launch's rows: a row chunk's scales
  // never reach past the caller's array)
  const uint32_t s_bytes = ((uint32_t)p.sfa_ld * (uint32_t)((UE ? KW : KB) - 1) + (uint32_t)rows) * 4u;
  const uint32_t sb_bytes = KG ? (uint32_t)N * (uint32_t)KB * 4u : 0u;  // K-grouped beta [KB][N]
  const __amdgpu_buffer_rsrc_t rd = F32OUT ? make_rsrc(p.Dacc, (uint32_t)rows * (uint32_t)N * 4u)
                                        : make_rsrc(p.D, (uint32_t)rows * (uint32_t)N * 2u);
  // accumulating form: C (a null C reads as zeros through a zero-length range)
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.Cacc, ACC && p.Cacc ? (uint32_t)rows * (uint32_t)N * 4u : 0u);

  // DMA lanes: instruction i of this wave fills LDS rows 64 i + 8 wave + lane / 8;
  // lane chunk (lane % 8) of row r holds K chunk (lane % 8) ^ (r % 8).  B rows
  // enter LDS permuted (row 16 j + i of a 64-row block holds weight row
  // (i / 4) * 16 + 4 j + i % 4 of it) so each lane ends with 16 consecutive
  // output columns of one row.
  const int dma_chunk = ((lane & 7) ^ ((lane >> 3) & 7)) << 4;
  const int a_loc = 8 * wave + (lane >> 3);
  const int b_perm = ((a_loc & 15) >> 2) * 16 + 4 * (a_loc >> 4) + (a_loc & 3);

  const int q16 = lane & 15;
  const uint32_t fr_lo = (uint32_t)(q16 * 128 + ((q ^ (lane & 7)) << 4));
  const uint32_t fr_hi = (uint32_t)(q16 * 128 + (((q + 4) ^ (lane & 7)) << 4));
  const uint32_t a_row0 = (uint32_t)(wm * 64 * 128);
  const uint32_t b_row0 = (uint32_t)(wn * 64 * 128);

#define PS_SLOT(st) ((st) == 0 ? slot0 : ((st) == 1 ? slot1 : slot2))
#define PS_SA(st) (PS_SLOT(st))
#define PS_SB(st) (PS_SLOT(st) + BM * 128)
#define PS_SS(st) (reinterpret_cast<float*>(PS_SLOT(st) + SLOT_S))

  // ---- issue pointer: iteration j + 3 of this workgroup's sequence.  Its
  // per-lane source offsets change only with its tile (rows outside the tile
  // get an offset past the buffer end); the K block enters through soffset.
  // K-grouped: waves 4 and 5 load beta of the tile's columns instead of alpha
  const bool bwave = KG && (wave == 4 || wave == 5);
  int is_seg = 0;
  Seg is_t = seg_of(0);
  int is_kb = is_t.kb_lo;
  uint32_t is_aoff[A_INS];
  uint32_t is_boff[B_INS];
  uint32_t is_soff;
  const uint8_t* is_aptr = p.A;    // the segment's group of A rows (masked)
  const uint8_t* is_bptr = p.B;    // the segment's expert's weights
  const float* is_sptr = p.sfa;    // the segment's group of alpha (masked)
  auto is_setup = [&]() {
    const int agrp = KG ? 0 : is_t.grp;  // K-grouped: A and alpha are shared by all groups
    is_aptr = p.A + (size_t)agrp * (size_t)rows * (size_t)K;
    is_sptr = p.sfa + (size_t)agrp * (size_t)(UE ? KW : KB) * (size_t)rows;
    is_bptr = p.B + (size_t)is_t.bgrp * (size_t)N * (size_t)K;
    const int arow = is_t.mt * BM;
    const int brow = is_t.nt * BN;
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int r = 64 * i + a_loc;
      is_aoff[i] = r < is_t.row_limit ? (uint32_t)(arow + r) * (uint32_t)K + dma_chunk : kOOB;
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      const int c = 64 * i + b_perm;
      is_boff[i] = is_t.nt * BN + c < N ? (uint32_t)(brow + c) * (uint32_t)K + dma_chunk : kOOB;
    }
    // scale lanes: alpha of the tile's rows that exist; beta (K-grouped) of
    // its columns below N; every other lane addresses past the range
    const int srow = wave * 64 + lane;
    is_soff = srow < BM && srow < is_t.row_limit ? (uint32_t)((is_t.mt * BM + srow) * 4) : kOOB;
    if (KG && bwave) {
      const int scol = is_t.nt * BN + (wave - 4) * 64 + lane;
      is_soff = scol < N ? (uint32_t)(scol * 4) : kOOB;
    }
  };
  is_setup();

  // Loads of the issue pointer's block into slot st_: PS_ISSUE_BEGIN selects
  // the ranges (zero-length past the last iteration, so those loads return
  // zeros; selected without a branch), PS_ISSUE_LOAD(st_, n) issues load n
  // (A_INS A loads, B_INS B loads, then alpha), PS_ISSUE_END advances the
  // pointer.  The three must share one scope.
#define PS_ISSUE_BEGIN()                                                                                   \
  const bool in_ = is_seg < nseg;                                                                          \
  const bool ld_ = in_ && !(KG && is_t.zero);                                                              \
  const __amdgpu_buffer_rsrc_t ra_ = make_rsrc(is_aptr, ld_ ? a_bytes : 0u);                               \
  const __amdgpu_buffer_rsrc_t rb_ = make_rsrc(is_bptr, ld_ ? b_bytes : 0u);                               \
  const __amdgpu_buffer_rsrc_t rs_ = bwave ? make_rsrc(p.sfb, ld_ ? sb_bytes : 0u)                         \
                                           : make_rsrc(is_sptr, ld_ ? s_bytes : 0u);                       \
  const int ks_ = is_kb << 7
#define PS_ISSUE_LOAD(st_, bs_, n_)                                                                        \
  do {                                                                                                     \
    if ((n_) < A_INS)                                                                                      \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_, (DG_LDS void*)(PS_SA(st_) + ((n_) * NWAVES + wave) * 1024), \
                                               16, is_aoff[(n_) < A_INS ? (n_) : 0], ks_, 0, 0);           \
    else if ((n_) < A_INS + B_INS)                                                                         \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb_,                                                        \
                                               (DG_LDS void*)(PS_SB(st_) + ((n_) - A_INS) * NWAVES * 1024 + wave * 1024), \
                                               16, is_boff[(n_) < A_INS + B_INS && (n_) >= A_INS ? (n_) - A_INS : 0], ks_, 0, \
                                               NT ? kStream : 0);                                          \
    else                                                                                                   \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                            \
          rs_, (DG_LDS void*)(bwave ? &bring[KG ? (bs_) : 0][(wave - 4) * 64] : PS_SS(st_) + wave * 64), 4,     \
          is_soff, (UE ? (is_kb >> 2) : is_kb) * (bwave ? N : p.sfa_ld) * 4, 0, 0);                         \
  } while (0)
#define PS_ISSUE_END()                                                                                     \
  do {                                                                                                     \
    if (in_ && ++is_kb == is_t.kb_hi) {                                                                    \
      if (++is_seg < nseg) {                                                                               \
        is_t = seg_of(is_seg);                                                                             \
        is_kb = is_t.kb_lo;                                                                                \
        is_setup();                                                                                        \
      }                                                                                                    \
    }                                                                                                      \
  } while (0)
#define PS_ISSUE(st_, bs_)                                                                                 \
  do {                                                                                                     \
    PS_ISSUE_BEGIN();                                                                                      \
    _Pragma("unroll") for (int n_ = 0; n_ < L_BLOCK; ++n_) PS_ISSUE_LOAD(st_, bs_, n_);                   \
    PS_ISSUE_END();                                                                                        \
  } while (0)

  int J = n_dp * KB;  // iterations of this workgroup
  if constexpr (KG) {
    J = 0;
    for (int s = 0; s < nseg; ++s) {
      const Seg t = seg_of(s);
      J += t.kb_hi - t.kb_lo;
    }
  }
  if (has_tail) {
    const Seg t = seg_of(n_dp);
    J += t.kb_hi - t.kb_lo;
  }

  // ---- compute pointer: iteration j
  int cp_seg = 0;
  Seg cp_t = seg_of(0);
  int cp_kb = cp_t.kb_lo;
  const DG_CONST float* sfb_w;
  auto cp_setup = [&]() {
    int nblk = (cp_t.nt * BN + wn * 64) >> 7;
    nblk = nblk < NB ? nblk : NB - 1;
    const uint64_t a = reinterpret_cast<uint64_t>(p.sfb + ((int64_t)cp_t.bgrp * NB + nblk) * (UE ? KW : KB));
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    sfb_w = (const DG_CONST float*)(((uint64_t)hi << 32) | lo);
  };
  cp_setup();

  f32x4 u[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) u[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // bf16 output of a finished tile, from u: for row tile i, lane l holds
  // output row wm*64 + 16 i + l % 16 and its 16 consecutive columns
  // wn*64 + q*16 + [0, 16) (two 16-byte stores; lanes outside the tile store
  // past the buffer end).  A tile that finishes in the main loop stays in u
  // until the next iteration's barrier has passed; its stores are then issued
  // ahead of that iteration's loads, so a whole iteration passes before a load
  // wait can depend on their completion.  (st_row0, st_col0, st_rows) locate
  // the tile.
  bool pend = false;
  int st_row0 = 0, st_col0 = 0, st_rows = 0, st_grp = 0;
  uint32_t st_m[4] = {~0u, ~0u, ~0u, ~0u};  // contiguous: rows tagged with the tile's expert
#define PS_MARK_TILE()                                                                                     \
  do {                                                                                                     \
    st_row0 = cp_t.mt * BM; /* masked: D of group st_grp from its own base */                            \
    st_col0 = cp_t.nt * BN;                                                                                \
    st_rows = cp_t.row_limit;                                                                              \
    st_grp = cp_t.grp;                                                                                     \
    if (FORM == kContiguous) {                                                                             \
      _Pragma("unroll") for (int w_ = 0; w_ < 4; ++w_) st_m[w_] = __builtin_amdgcn_readfirstlane(seg_mask[cp_seg][w_]); \
    }                                                                                                      \
  } while (0)
#define PS_OUT_OFF(i_)                                                                                     \
  ([&]() -> uint32_t {                                                                                     \
    const int gc0_ = st_col0 + wn * 64 + q * 16;                                                           \
    const int r_ = wm * 64 + (i_) * 16 + q16;                                                              \
    const bool tag_ = FORM != kContiguous || ((st_m[r_ >> 5] >> (r_ & 31)) & 1u);                          \
    return (r_ < st_rows && gc0_ < N && tag_) ? ((uint32_t)(st_row0 + r_) * (uint32_t)N + gc0_) * 2u : kOOB; \
  }())
  // Accumulating forms: fp32 outputs, 64 bytes per lane and row tile (byte
  // offsets twice the bf16 ones); with C given, every C load of the tile is
  // issued before the first store (C may be D itself), then the sums are
  // stored; without C, u is stored.  K-grouped: C and D of the tile's group,
  // one [rows][N] matrix each.
#define PS_STORE_U()                                                                                       \
  do {                                                                                                     \
    if constexpr (F32OUT) {                                                                                \
      const size_t gof_ = KG ? (size_t)st_grp * (size_t)rows * (size_t)N : 0;                              \
      const __amdgpu_buffer_rsrc_t rd_ = KG ? make_rsrc(p.Dacc + gof_, (uint32_t)rows * (uint32_t)N * 4u) : rd; \
      const __amdgpu_buffer_rsrc_t rc_ =                                                                   \
          KG ? make_rsrc(p.Cacc + (p.Cacc ? gof_ : 0), p.Cacc ? (uint32_t)rows * (uint32_t)N * 4u : 0u) : rc;   \
      uint32_t o_[TM];                                                                                     \
      f32x4 c_[TM][TN];                                                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) {                                                  \
        const uint32_t b_ = PS_OUT_OFF(i_);                                                                \
        o_[i_] = b_ == kOOB ? kOOB : 2u * b_;                                                              \
        _Pragma("unroll") for (int j_ = 0; j_ < TN; ++j_)                                                  \
          c_[i_][j_] = HASC ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rc_, o_[i_] + 16u * j_, 0, 0)) \
                            : f32x4{0.f, 0.f, 0.f, 0.f};                                                   \
      }                                                                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_)                                                    \
        _Pragma("unroll") for (int j_ = 0; j_ < TN; ++j_)                                                  \
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, u[i_][j_] + c_[i_][j_]), rd_,   \
                                                 o_[i_] + 16u * j_, 0, 0);                                 \
    } else {                                                                                               \
      const __amdgpu_buffer_rsrc_t rdm_ =                                                                  \
          FORM == kMasked ? make_rsrc(p.D + (size_t)st_grp * (size_t)rows * (size_t)N, (uint32_t)rows * (uint32_t)N * 2u) : rd; \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) {                                                  \
        const uint32_t off_ = PS_OUT_OFF(i_);                                                              \
        uint32_t w_[8];                                                                                    \
        _Pragma("unroll") for (int j_ = 0; j_ < TN; ++j_) {                                                \
          w_[2 * j_] = pack_bf16x2(u[i_][j_][0], u[i_][j_][1]);                                            \
          w_[2 * j_ + 1] = pack_bf16x2(u[i_][j_][2], u[i_][j_][3]);                                        \
        }                                                                                                  \
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{w_[0], w_[1], w_[2], w_[3]}, rdm_, off_, 0, 0);       \
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{w_[4], w_[5], w_[6], w_[7]}, rdm_,                    \
                                               off_ == kOOB ? kOOB : off_ + 16u, 0, 0);                    \
      }                                                                                                    \
    }                                                                                                      \
  } while (0)

#define PS_FRAG(dst_, base_, off_)                                                                         \
  do {                                                                                                     \
    const uint4 lo_ = *reinterpret_cast<const uint4*>((base_) + fr_lo + (off_));                          \
    const uint4 hi_ = *reinterpret_cast<const uint4*>((base_) + fr_hi + (off_));                          \
    dst_ = i32x8{(int)lo_.x, (int)lo_.y, (int)lo_.z, (int)lo_.w, (int)hi_.x, (int)hi_.y, (int)hi_.z, (int)hi_.w}; \
  } while (0)

  // this wave's fragments and row scales of the iteration held in slot st_
#define PS_LOAD_FRAGS(st_, AF, BF, AL)                                                                     \
  do {                                                                                                     \
    const uint8_t* as_ = PS_SA(st_) + a_row0;                                                              \
    const uint8_t* bs_ = PS_SB(st_) + b_row0;                                                              \
    _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) {                                                    \
      PS_FRAG(AF[i_], as_, i_ * 2048);                                                                     \
      AL[i_] = BF16 ? 1.f : PS_SS(st_)[wm * 64 + i_ * 16 + q16];                                           \
    }                                                                                                      \
    _Pragma("unroll") for (int j_ = 0; j_ < TN; ++j_) PS_FRAG(BF[j_], bs_, j_ * 2048);                    \
  } while (0)

  // BF16 mode: the products of one iteration accumulate straight into u.  A
  // fragment's 16 bytes at chunk q hold K elements 8 q .. 8 q + 7 of the
  // block's first 32, those at chunk q + 4 the same of its second 32 (both
  // operands use the same mapping, so the dot products are the block's), so
  // each 16x16 tile takes two 16x16x32 bf16 MFMAs: all first halves, then all
  // second halves (each depends on its first half 16 MFMAs earlier).  The
  // next iteration's fragment reads and the block's loads are interleaved as
  // in the FP8 path.
#define PS_COMPUTE_BF16(st_, bs_, AF, BF, AN, BN_)                                                         \
  do {                                                                                                     \
    const uint8_t* nsl_ = PS_SLOT(((st_) + 1) % 3);                                                        \
    uint4 nlo_[TM + TN], nhi_[TM + TN];                                                                    \
    _Pragma("unroll") for (int k_ = 0; k_ < 2 * TM * TN; ++k_) {                                           \
      const int t_ = k_ % (TM * TN);                                                                       \
      const int i_ = t_ % TM;                                                                              \
      const int j_ = t_ / TM;                                                                              \
      const i32x4 av_ = k_ < TM * TN ? i32x4{AF[i_][0], AF[i_][1], AF[i_][2], AF[i_][3]}                   \
                                     : i32x4{AF[i_][4], AF[i_][5], AF[i_][6], AF[i_][7]};                  \
      const i32x4 bv_ = k_ < TM * TN ? i32x4{BF[j_][0], BF[j_][1], BF[j_][2], BF[j_][3]}                   \
                                     : i32x4{BF[j_][4], BF[j_][5], BF[j_][6], BF[j_][7]};                  \
      u[i_][j_] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bv_),                \
                                                         __builtin_bit_cast(bf16x8, av_), u[i_][j_], 0, 0, 0); \
      if (k_ < L_BLOCK) PS_ISSUE_LOAD(st_, bs_, k_);                                                       \
      if (k_ < 2 * (TM + TN)) {                                                                            \
        const int f_ = k_ >> 1; /* fragment: A 0..TM-1, then B */                                          \
        const uint32_t o_ = (f_ < TM ? a_row0 + f_ * 2048 : BM * 128 + b_row0 + (f_ - TM) * 2048) +        \
                            ((k_ & 1) ? fr_hi : fr_lo);                                                    \
        if (k_ & 1) nhi_[f_] = *reinterpret_cast<const uint4*>(nsl_ + o_);                                 \
        else nlo_[f_] = *reinterpret_cast<const uint4*>(nsl_ + o_);                                        \
      }                                                                                                    \
      __builtin_amdgcn_sched_barrier(0);                                                                   \
    }                                                                                                      \
    _Pragma("unroll") for (int f_ = 0; f_ < TM + TN; ++f_) {                                               \
      const i32x8 v8_ = i32x8{(int)nlo_[f_].x, (int)nlo_[f_].y, (int)nlo_[f_].z, (int)nlo_[f_].w,          \
                              (int)nhi_[f_].x, (int)nhi_[f_].y, (int)nhi_[f_].z, (int)nhi_[f_].w};         \
      if (f_ < TM) AN[f_] = v8_;                                                                           \
      else BN_[f_ - TM] = v8_;                                                                             \
    }                                                                                                      \
  } while (0)

  // The products and promotions of one iteration, with the next iteration's
  // fragment reads from slot (st_ + 1) % 3 interleaved.  Dense: a fixed
  // order of 16 steps, each one MFMA (B fragment j = k / 4, A fragment
  // i = k % 4), one 16-byte LDS read of the next fragments (and, in the first steps,
  // one of the block's loads) and the four promotion FMAs of the MFMA three
  // steps back, so the LDS reads and the FMAs
  // overlap the matrix cores.
#define PS_COMPUTE(st_, bs_, br_, AF, BF, AL, AN, BN_, ALN)                                                \
  do {                                                                                                     \
    float sc_[TM];                                                                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) sc_[i_] = AL[i_] * beta_;                            \
    if constexpr (BF16) {                                                                                  \
      PS_COMPUTE_BF16(st_, bs_, AF, BF, AN, BN_);                                                          \
      (void)sc_;                                                                                           \
    } else {                                                                                               \
      const uint8_t* nsl_ = PS_SLOT(((st_) + 1) % 3);                                                      \
      uint4 nlo_[TM + TN], nhi_[TM + TN];                                                                  \
      f32x4 t_[TM * TN];                                                                                   \
      f32x4 bt_[2]; /* K-grouped: beta of the 4 columns of fragment j, two j in flight */                  \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) ALN[i_] = PS_SS(((st_) + 1) % 3)[wm * 64 + i_ * 16 + q16]; \
      _Pragma("unroll") for (int k_ = 0; k_ < TM * TN + 3; ++k_) {                                         \
        if (k_ < TM * TN) {                                                                                \
          if constexpr (UE) { /* alpha and beta applied, and the scaled block product added to the */      \
            /* accumulator, by the matrix cores (exact powers of two): the promotion in one instruction */  \
            u[k_ % TM][k_ / TM] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                         \
                BF[k_ / TM], AF[k_ % TM], u[k_ % TM][k_ / TM], 0, 0, 0, bcode_, 0,                          \
                __builtin_bit_cast(int, AL[k_ % TM]) >> ash_);                                             \
          } else {                                                                                         \
            t_[k_] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(BF[k_ / TM], AF[k_ % TM], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0); \
          }                                                                                                \
          if (KG && k_ % TM == 0)                                                                          \
            bt_[(k_ / TM) & 1] = *reinterpret_cast<const f32x4*>(&bring[KG ? (br_) : 0][KG ? wn * 64 + q * 16 + 4 * (k_ / TM) : 0]); \
          if (k_ < L_BLOCK) PS_ISSUE_LOAD(st_, bs_, k_); /* the block's loads, spread over the first steps */ \
          const int f_ = k_ >> 1; /* fragment: A 0..TM-1, then B */                                        \
          const uint32_t o_ = (f_ < TM ? a_row0 + f_ * 2048 : BM * 128 + b_row0 + (f_ - TM) * 2048) +      \
                              ((k_ & 1) ? fr_hi : fr_lo);                                                  \
          if (k_ & 1) nhi_[f_] = *reinterpret_cast<const uint4*>(nsl_ + o_);                               \
          else nlo_[f_] = *reinterpret_cast<const uint4*>(nsl_ + o_);                                      \
        }                                                                                                  \
        if (k_ >= 3) {                                                                                     \
          const int kk_ = k_ - 3;                                                                          \
          f32x4& uk_ = u[kk_ % TM][kk_ / TM];                                                              \
          if constexpr (!UE) {                                                                             \
            if constexpr (KG) t_[kk_] *= bt_[(kk_ / TM) & 1];                                              \
            _Pragma("unroll") for (int v_ = 0; v_ < 4; ++v_)                                               \
              uk_[v_] = __builtin_fmaf(t_[kk_][v_], sc_[kk_ % TM], uk_[v_]);                               \
          }                                                                                                \
          /* keeps these FMAs in this step: instruction selection would sink them to the block's end */    \
          /* (UE8M0: pins the accumulator of the MFMA three steps back, which keeps the schedule) */       \
          asm volatile("" : "+v"(uk_));                                                                    \
        }                                                                                                  \
        __builtin_amdgcn_sched_barrier(0);                                                                 \
      }                                                                                                    \
      _Pragma("unroll") for (int f_ = 0; f_ < TM + TN; ++f_) {                                             \
        const i32x8 v8_ = i32x8{(int)nlo_[f_].x, (int)nlo_[f_].y, (int)nlo_[f_].z, (int)nlo_[f_].w,        \
                                (int)nhi_[f_].x, (int)nhi_[f_].y, (int)nhi_[f_].z, (int)nhi_[f_].w};       \
        if (f_ < TM) AN[f_] = v8_;                                                                         \
        else BN_[f_ - TM] = v8_;                                                                           \
      }                                                                                                    \
    }                                                                                                      \
  } while (0)

  // One iteration jj_ (slot st_ = jj_ % 3), see the header.  Fragments of
  // iteration jj_ (AF, BF, AL) were read during iteration jj_ - 1; those of
  // jj_ + 1 are read here (AN, BN_, ALN) while the matrix cores work.  The
  // wait for iteration jj_ + 1 counts loads only: loads complete in issue
  // order, so at most L_BLOCK outstanding operations means all loads up to
  // iteration jj_ + 1 have landed, whatever output stores are also in flight
  // (those only add to the count).  Iterations past this workgroup's last one
  // read zero operands (their loads address zero-length ranges) and a zero
  // scale, so their products add exactly nothing.
#define PS_STEP(c_, jj_, AF, BF, AL, AN, BN_, ALN)                                                         \
  do {                                                                                                     \
    constexpr int st_ = (c_) % 3;                                                                          \
    const bool live_ = (jj_) < J;                                                                          \
    const float beta_ = BF16 || KG || UE ? 1.f : (live_ ? sfb_w[cp_kb] : 0.f);                            \
    /* UE8M0: the iteration's codes sit in byte cp_kb % 4 of their packed words */                        \
    const int ash_ = 8 * (cp_kb & 3);                                                                      \
    const int bcode_ = UE && live_ ? __builtin_bit_cast(int, sfb_w[cp_kb >> 2]) >> ash_ : 0;              \
    (void)ash_;                                                                                            \
    (void)bcode_;                                                                                          \
    wait_vmcnt<L_BLOCK>();                                                                                 \
    wait_lgkmcnt0(); /* own reads of this slot done before anyone may refill it */                        \
    __builtin_amdgcn_s_barrier();                                                                          \
    if (pend) {                                                                                            \
      PS_STORE_U();                                                                                        \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_)                                                    \
        _Pragma("unroll") for (int j_ = 0; j_ < TN; ++j_) u[i_][j_] = f32x4{0.f, 0.f, 0.f, 0.f};           \
      pend = false;                                                                                        \
    }                                                                                                      \
    {                                                                                                      \
      PS_ISSUE_BEGIN();                                                                                    \
      PS_COMPUTE(st_, (c_ + 3) % 6, c_, AF, BF, AL, AN, BN_, ALN);                                         \
      PS_ISSUE_END();                                                                                      \
    }                                                                                                      \
    if (live_ && ++cp_kb == cp_t.kb_hi && cp_t.tail < 0) { /* a whole tile is done */                     \
      PS_MARK_TILE();                                                                                      \
      pend = true;                                                                                         \
      if (++cp_seg < nseg) {                                                                               \
        cp_t = seg_of(cp_seg);                                                                             \
        cp_kb = cp_t.kb_lo;                                                                                \
        cp_setup();                                                                                        \
      }                                                                                                    \
    }                                                                                                      \
  } while (0)

  i32x8 afX[TM], bfX[TN], afY[TM], bfY[TN];
  float alX[TM], alY[TM];
  // prologue: iterations 0, 1, 2 into slots 0, 1, 2; fragments of iteration 0
  PS_ISSUE(0, 0);
  PS_ISSUE(1, 1);
  PS_ISSUE(2, 2);
  wait_vmcnt<2 * L_BLOCK>();  // iteration 0 landed (this wave's part)
  __builtin_amdgcn_s_barrier();
  PS_LOAD_FRAGS(0, afX, bfX, alX);
  // iterations, padded to whole cycles of ring slots and fragment registers;
  // a tail piece (always this workgroup's last segment) leaves the loop with
  // its partial in u
  for (int j = 0; j < J; j += 6) {
    PS_STEP(0, j, afX, bfX, alX, afY, bfY, alY);
    PS_STEP(1, j + 1, afY, bfY, alY, afX, bfX, alX);
    PS_STEP(2, j + 2, afX, bfX, alX, afY, bfY, alY);
    PS_STEP(3, j + 3, afY, bfY, alY, afX, bfX, alX);
    PS_STEP(4, j + 4, afX, bfX, alX, afY, bfY, alY);
    PS_STEP(5, j + 5, afY, bfY, alY, afX, bfX, alX);
  }
  if (pend) PS_STORE_U();
  wait_vmcnt<0>();  // no LDS writes or stores in flight past this point
  wait_lgkmcnt0();

#undef PS_STEP
#undef PS_COMPUTE
#undef PS_COMPUTE_BF16
#undef PS_ISSUE
#undef PS_ISSUE_BEGIN
#undef PS_ISSUE_LOAD
#undef PS_ISSUE_END
#undef PS_LOAD_FRAGS
#undef PS_FRAG
#undef PS_SA
#undef PS_SB
#undef PS_SS
#undef PS_SLOT

  if (has_tail) {
    // K-split tail tile: fp32 partial in fragment order (piece pc of tail
    // tile s, wave w, fragment (i, j), lane l at byte
    // (((s * P + pc) * 8 + w) * 16 + i * 4 + j) * 1024 + 16 l after the
    // counter area); the last piece sums all pieces' partials in piece order.
    // Ordering: the partial stores and loads carry sc1 -- the compiler's
    // lowering of relaxed agent-scope atomic stores and loads on gfx950 -- so
    // they are coherent across the XCDs' L2 caches.  Every wave waits
    // (vmcnt(0)) until its stores are acknowledged at that coherence point,
    // the barrier then orders all of them before the relaxed counter
    // increment, and the last piece issues its loads only after its own
    // increment has returned (so after every other piece's increment, which
    // followed that piece's acknowledged stores).  An agent-scope release /
    // acquire would add an L2 write-back / invalidate, needed only for data
    // cached non-coherently, which these accesses never are.
    const uint32_t frag_bytes = (uint32_t)TM * TN * 1024u;
    const uint32_t tile_bytes = (uint32_t)NWAVES * frag_bytes;
    // counters at the workspace start, partials after them
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(reinterpret_cast<uint8_t*>(p.ws) + kWsCounterBytes, (uint32_t)p.sk_tiles * (uint32_t)P * tile_bytes);
    const uint32_t w_off = (uint32_t)(cp_t.tail * P) * tile_bytes + (uint32_t)wave * frag_bytes + (uint32_t)lane * 16u;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, u[i][j]), rw,
                                               w_off + (uint32_t)(i * TN + j) * 1024u,
                                               (uint32_t)cp_t.piece * tile_bytes, kCoherent);
    wait_vmcnt<0>();
    __syncthreads();
    unsigned int* counters = reinterpret_cast<unsigned int*>(p.ws);
    if (tid == 0)
      last_piece = __hip_atomic_fetch_add(&counters[cp_t.tail], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (unsigned int)(P - 1);
    __syncthreads();
    if (!last_piece) return;
#define PS_LDP(pc_, i_, j_)                                                                                \
  __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(                                         \
                                rw, w_off + (uint32_t)((i_) * TN + (j_)) * 1024u, (uint32_t)(pc_) * tile_bytes, kCoherent))
    // two pieces' loads in flight at a time, added in piece order
    for (int pc0 = 0; pc0 < P; pc0 += 2) {
      f32x4 t0[TM][TN], t1[TM][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          t0[i][j] = PS_LDP(pc0, i, j);
          if (pc0 + 1 < P) t1[i][j] = PS_LDP(pc0 + 1, i, j);
        }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          u[i][j] = pc0 == 0 ? t0[i][j] : u[i][j] + t0[i][j];
          if (pc0 + 1 < P) u[i][j] += t1[i][j];
        }
    }
#undef PS_LDP
    if (tid == 0)  // ready for the next call on this workspace
      __hip_atomic_store(&counters[cp_t.tail], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    PS_MARK_TILE();
    PS_STORE_U();
  }
#undef PS_MARK_TILE
#undef PS_STORE_U
#undef PS_OUT_OFF
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace

size_t persistent_workspace_bytes(int sk_tiles, int sk_pieces) {
  if (sk_tiles <= 0 || sk_pieces <= 1) return 0;
  // the counter area, then fp32 partials of 256 x 128 tiles
  return kWsCounterBytes + (size_t)sk_tiles * sk_pieces * 256 * 128 * 4;
}

hipError_t launch_gemm_persistent(int mode, int grid, const GemmParams& p, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid), t(512);
  const bool c = p.Cacc != nullptr;
  const bool nt = p.m_tiles == 1;  // masked: one 128-row tile per expert
  if (mode == kMasked && nt)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kMasked, false, true>), g, t, 0, stream, p);
  else if (mode == kMasked)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kMasked, false, false>), g, t, 0, stream, p);
  else if (mode == kDenseBf16)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kDenseBf16, false, false>), g, t, 0, stream, p);
  else if (mode == kDenseAcc && c)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kDenseAcc, true, false>), g, t, 0, stream, p);
  else if (mode == kDenseAcc)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kDenseAcc, false, false>), g, t, 0, stream, p);
  else if (mode == kKGrouped && c)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kKGrouped, true, false>), g, t, 0, stream, p);
  else if (mode == kKGrouped)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kKGrouped, false, false>), g, t, 0, stream, p);
  else if (mode == kContiguous)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kContiguous, false, false>), g, t, 0, stream, p);
  else if (mode == kDenseUe8m0)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kDenseUe8m0, false, false>), g, t, 0, stream, p);
  else if (mode == kContiguousUe8m0)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kContiguousUe8m0, false, false>), g, t, 0, stream, p);
  else if (mode == kMaskedUe8m0 && nt)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kMaskedUe8m0, false, true>), g, t, 0, stream, p);
  else if (mode == kMaskedUe8m0)
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kMaskedUe8m0, false, false>), g, t, 0, stream, p);
  else
    hipLaunchKernelGGL((fp8_gemm_persistent_kernel<kDense, false, false>), g, t, 0, stream, p);
  return hipGetLastError();
}

}  // namespace dg
