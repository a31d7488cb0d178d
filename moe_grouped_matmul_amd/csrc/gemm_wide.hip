// Wide-tile persistent block-scaled FP8 GEMM for gfx950: one 512-thread
// workgroup per CU walks 256 x 256 output tiles.  Modes: the dense form
// (bf16 output), its UE8M0-scale, BF16-operand and accumulating (fp32
// D = C + A . B^T) variants, the M-grouped contiguous form and the K-grouped
// form (fp32 per-group output).
//
// The computation is the one of Lesson 13 (hpc.payai.win), Fig. 13-1 and its
// closed-form equation: every 128-wide K block's fp8 partial product of a
// tile is formed by the matrix cores and promoted into an fp32 accumulator
// with alpha[row, k] * beta[k]; the epilogue rounds to bf16.
//
// Why a second persistent kernel: with 256 x 128 tiles each CU streams 48 KB
// of operands per 8.4 MFLOP and the large shapes run at the rate one CU's
// L2 request path sustains.  A 256 x 256 tile streams 64 KB per 16.8 MFLOP,
// a third fewer bytes per flop.  Its cost is registers and LDS:
//   * eight waves (two per SIMD), each a 64 x 128 sub-tile of 4 x 8
//     v_mfma_f32_16x16x128_f8f6f4 tiles, 128 accumulator registers;
//   * a two-slot LDS ring (64 KB of operands + 2 KB of alpha per slot; three
//     slots would not fit): the loads of iteration j + 1 go to the other slot
//     while iteration j computes, one s_barrier per iteration publishes them;
//   * fragments are read from the slot of the running iteration: the four
//     A fragments and the row scales after the barrier, the B fragments one
//     ahead of their four MFMAs (two B registers sets alternate);
//   * the promotion FMAs of each MFMA run three MFMAs later, as in the
//     256 x 128 kernel (gemm_persist.hip), whose operand layout, swizzle, B
//     row permutation and deferred bf16 store this kernel shares.
// Tile walk: lockstep rounds of one tile per workgroup (m-grouped ids),
// each XCD a contiguous run of the round.  No K split: used where the tiles
// fill the CUs in whole or nearly whole rounds.
//
// UE8M0 scales (dense and contiguous): alpha and beta are powers of two given
// by their exponent bytes, four K blocks per 32-bit word (as in
// gemm_persist.hip).
// The matrix cores apply them (v_mfma_scale_f32_16x16x128_f8f6f4: beta's byte
// for the B operand, each row's alpha byte for the A operand), which is exact,
// and accumulate the scaled block product into the tile's fp32 accumulator:
// the promotion is the MFMA itself (bit for bit the separate fp32 add, as the
// accumulator input is added with one rounding after the products).
//
// BF16 operands (plain GEMM, no scales): a K block is 64 bf16 = 128 bytes
// per row, so LDS rows, swizzle, DMA and fragment reads are those of the fp8
// path.  A fragment's chunk q holds K elements 8 q .. 8 q + 7 of the block's
// first 32, chunk q + 4 the same of its second 32 (both operands map them
// alike), so each 16 x 16 tile takes two v_mfma_f32_16x16x32_bf16 straight
// into the accumulator: the 32 first halves (B half fragments streamed one
// ahead), then the 32 second halves, each 32 MFMAs after its first half.
//
// Accumulating form (fp32 D = C + A . B^T, C optional and possibly D itself):
// a finished tile is written row tile by row tile, the C fragments of the
// next row tile loaded before the current one is stored (two in flight;
// distinct rows, so C = D in place stays correct).
//
// K-grouped form (MoE weight gradient, fp32 D[g] = C[g] + A[:, seg g] .
// B[:, seg g]^T): every workgroup reads the group lengths on the device and
// builds the first K block of each group; the tiles of all groups are walked
// in rounds of one tile per workgroup (XCD-contiguous inside a round), each
// tile over its group's K blocks only (a group without blocks runs one
// iteration over zeros, so its tiles still store C).  Waves 4..7 load the
// per-column beta of the tile's 256 columns where the other forms have no
// alpha rows, and the promotion scales each product by its columns' beta
// before the row's alpha.
//
// M-grouped contiguous form (Lesson 13, Fig. 13-3, contiguous layout): only
// aligned 128-row blocks are guaranteed to hold one expert, so a 256-row tile
// may straddle two.  Every workgroup reads m_indices of its own tiles at
// start and lists its passes in LDS: a tile whose two halves belong to one
// expert (or whose other half has none) is one pass; a tile straddling two
// experts is two passes, each with its expert's weights and storing only the
// rows tagged with that expert; a tile without a valid index is none.  A
// pass whose rows lie in one 128-row half runs the MFMAs of that half's four
// waves only (each SIMD holds one wave of each half) and loads no A rows of
// the other half, so a straddling tile costs about one full pass.  A pass
// loads the A rows tagged with its expert only.

#include "dg_internal.hpp"
#include "gemm_common.hpp"

namespace dg {
namespace {

constexpr int kWideRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family
constexpr uint32_t kWideOOB = 0xFFFFFF00u;  // an offset past every buffer range used here
constexpr int kWideMaxGroups = 1024;        // groups the K-grouped prefix table holds

typedef unsigned int wu32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 wbf16x8 __attribute__((ext_vector_type(8)));
typedef int wi32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wide_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kWideRsrcWord3);
}

template <int MODE, bool HASC>
__global__ void __launch_bounds__(512) fp8_gemm_wide_kernel(GemmParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(MODE == kDense || MODE == kContiguous || MODE == kDenseUe8m0 || MODE == kContiguousUe8m0 ||
                    MODE == kDenseBf16 || MODE == kDenseAcc || MODE == kKGrouped,
                "modes of the wide kernel");
  constexpr bool KG = MODE == kKGrouped;     // groups along K, per-column beta, fp32 D[g] = C[g] + ...
  constexpr bool ACC = MODE == kDenseAcc || KG;  // fp32 output D = C + A . B^T
  constexpr bool CONTIG = MODE == kContiguous || MODE == kContiguousUe8m0;
  // UE8M0 codes, applied by the matrix cores' block scaling (dense and contiguous)
  constexpr bool UE = MODE == kDenseUe8m0 || MODE == kContiguousUe8m0;
  constexpr bool BF16 = MODE == kDenseBf16;  // bf16 operands, no scales, no promotion
  constexpr int MAXT = kWideMaxContigTiles;  // tiles per workgroup the contiguous pass table holds
  constexpr int WGN = 2;
  constexpr int TM = 4;
  constexpr int TN = 8;
  constexpr int BM = 256;
  constexpr int BN = 256;
  constexpr int NWAVES = 8;
  constexpr int A_INS = BM / 8 / NWAVES;      // 1 KB (8-row) loads per wave per K block
  constexpr int B_INS = BN / 8 / NWAVES;
  constexpr int L_BLOCK = A_INS + B_INS + (BF16 ? 0 : 1);  // + one alpha load per wave
  constexpr int GM = 4;                       // m-tiles per tile group of the walk
  constexpr int SLOT_S = (BM + BN) * 128;
  constexpr int SLOT_BYTES = SLOT_S + NWAVES * 64 * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[SLOT_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[SLOT_BYTES];
  // contiguous: passes of this workgroup (tile id, expert, tagged-row mask)
  // and, per tile, its pass count then first pass
  __shared__ int pass_tile[CONTIG ? 2 * MAXT : 1];
  __shared__ int pass_exp[CONTIG ? 2 * MAXT : 1];
  __shared__ int pass_half[CONTIG ? 2 * MAXT : 1];  // bit h: rows of 128-row half h take part
  __shared__ uint32_t pass_mask[CONTIG ? 2 * MAXT : 1][8];
  __shared__ int tile_np[CONTIG ? MAXT + 1 : 1];
  __shared__ int kpref[KG ? kWideMaxGroups + 1 : 1];  // K-grouped: first K block of each group
  // bf16 output outside the contiguous form: each wave's 2 KB transpose buffer of the tile store
  __shared__ __attribute__((aligned(16))) uint8_t stage[!ACC && !CONTIG ? NWAVES * 2048 : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN;
  const int wn = wave % WGN;
  const int q = lane >> 4;
  const int q16 = lane & 15;
  const int b = (int)blockIdx.x;
  const int G = (int)gridDim.x;

  const int K = BF16 ? 2 * p.K : p.K;  // bytes per operand row
  const int N = p.N;
  const int KB = K >> 7;
  const int KW = (KB + 3) >> 2;  // UE8M0: packed words (four K blocks) per scale row
  const int NB = (N + 127) >> 7;
  const int rows = (int)p.rows;
  const int tpg = p.m_tiles * p.n_tiles;  // tiles per group (K-grouped) or in all
  const int T = KG ? p.G * tpg : tpg;
  const int n_dp = b < T ? (T - b + G - 1) / G : 0;  // tiles of this workgroup
  if (n_dp == 0) return;  // uniform over the workgroup
  if constexpr (KG) {
    // kpref[g] = first K block of group g: prefix of floor(ks / 128), clamped to KB
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
        if (g < p.G) kpref[g + 1] = carry + v < KB ? carry + v : KB;
        carry += __shfl(v, 63);
        carry = carry < KB ? carry : KB;
      }
      if (lane == 0) kpref[0] = 0;
    }
    __syncthreads();
  }
  // tile s of this workgroup: lockstep rounds of G consecutive tiles, each XCD
  // a contiguous run inside the round, so all XCDs work on neighbouring tiles
  // at any time (the contiguous form: the same few experts' weights).  Against
  // each XCD walking its own eighth of the tiles this measured 1035 -> 972 us
  // on the 8-expert 4096x7168 contiguous call and 114 -> 94 us on
  // 4096x32768x512 (its bf16 output is then written in one region at a time).
  auto dense_tile = [&](int s, int* mt, int* nt) { grouped_mn(round_tile(b, s, G, T), p.m_tiles, p.n_tiles, GM, mt, nt); };

  int nseg = n_dp;  // passes (dense: one per tile)
  if constexpr (CONTIG) {
    // m_indices of tile s's 256 rows: lane l holds rows 64 k + l, k < 4 (the
    // first two in the lower 128-row half); -1 for rows past M or indices
    // outside [0, G)
    auto tile_idx = [&](int s, int* v) {
      int mt, nt;
      dense_tile(s, &mt, &nt);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = mt * BM + 64 * k + lane;
        const int x = r < rows ? p.index[r] : -1;
        v[k] = x >= 0 && x < p.G ? x : -1;
      }
    };
    auto wave_max = [&](int x) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const int o = __shfl_xor(x, off);
        x = o > x ? o : x;
      }
      return x;
    };
    for (int s = wave; s < n_dp; s += NWAVES) {
      int v[4];
      tile_idx(s, v);
      const int e0 = wave_max(v[0] > v[1] ? v[0] : v[1]);
      const int e1 = wave_max(v[2] > v[3] ? v[2] : v[3]);
      if (lane == 0) tile_np[s] = (e0 < 0 && e1 < 0) ? 0 : ((e0 < 0 || e1 < 0 || e0 == e1) ? 1 : 2);
    }
    __syncthreads();
    if (wave == 0) {  // exclusive prefix of the pass counts (n_dp <= MAXT = 64)
      int c = lane < n_dp ? tile_np[lane] : 0;
      const int own = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(c, off);
        if (lane >= off) c += o;
      }
      if (lane < n_dp) tile_np[lane] = c - own;
      if (lane == 63) tile_np[MAXT] = c;
    }
    __syncthreads();
    for (int s = wave; s < n_dp; s += NWAVES) {
      int v[4];
      tile_idx(s, v);
      const int e0 = wave_max(v[0] > v[1] ? v[0] : v[1]);
      const int e1 = wave_max(v[2] > v[3] ? v[2] : v[3]);
      const int first = tile_np[s];
      const int np = (e0 < 0 && e1 < 0) ? 0 : ((e0 < 0 || e1 < 0 || e0 == e1) ? 1 : 2);
      for (int pp = 0; pp < np; ++pp) {
        const int e = np == 2 ? (pp == 0 ? e0 : e1) : (e0 > e1 ? e0 : e1);
        const int hm = (e0 == e ? 1 : 0) | (e1 == e ? 2 : 0);
        uint32_t m[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const unsigned long long bb = __ballot(v[k] == e);
          m[2 * k] = (uint32_t)bb;
          m[2 * k + 1] = (uint32_t)(bb >> 32);
        }
        if (lane == 0) {
          pass_tile[first + pp] = s;
          pass_exp[first + pp] = e;
          pass_half[first + pp] = hm;
#pragma unroll
          for (int w = 0; w < 8; ++w) pass_mask[first + pp][w] = m[w];
        }
      }
    }
    __syncthreads();
    nseg = __builtin_amdgcn_readfirstlane(tile_np[MAXT]);
    if (nseg == 0) return;  // no row of these tiles is tagged: nothing to store
  }
  int J = nseg * KB;  // iterations of this workgroup (K-grouped: counted below)

  // A, alpha and D of this launch and one expert's B are addressed with
  // 32-bit offsets from their bases (the expert's weights from its own
  // 64-bit base); alpha rows are sfa_ld apart
  const uint32_t a_bytes = (uint32_t)rows * (uint32_t)K;
  const uint32_t b_bytes = (uint32_t)N * (uint32_t)K;
  // (the last scale row ends after this launch's rows: a row chunk's scales
  // never reach past the caller's array)
  const uint32_t s_bytes = ((uint32_t)p.sfa_ld * (uint32_t)((UE ? KW : KB) - 1) + (uint32_t)rows) * 4u;
  const __amdgpu_buffer_rsrc_t rd = ACC ? wide_rsrc(p.Dacc, (uint32_t)rows * (uint32_t)N * 4u)
                                        : wide_rsrc(p.D, (uint32_t)rows * (uint32_t)N * 2u);
  const __amdgpu_buffer_rsrc_t rc = wide_rsrc(p.Cacc, HASC ? (uint32_t)rows * (uint32_t)N * 4u : 0u);

  // DMA lanes (as gemm_persist.hip): instruction i of this wave fills LDS rows
  // 64 i + 8 wave + lane / 8, lane chunk (lane % 8) of row r holding K chunk
  // (lane % 8) ^ (r % 8); B rows permuted inside each 64-row block so each
  // lane ends with 16 consecutive output columns of a 64-column half.
  const int dma_chunk = ((lane & 7) ^ ((lane >> 3) & 7)) << 4;
  const int a_loc = 8 * wave + (lane >> 3);
  const int b_perm = ((a_loc & 15) >> 2) * 16 + 4 * (a_loc >> 4) + (a_loc & 3);
  const uint32_t fr_lo = (uint32_t)(q16 * 128 + ((q ^ (lane & 7)) << 4));
  const uint32_t fr_hi = (uint32_t)(q16 * 128 + (((q + 4) ^ (lane & 7)) << 4));
  const uint32_t a_row0 = (uint32_t)(wm * 64 * 128);
  const uint32_t b_row0 = (uint32_t)(BM * 128 + wn * 128 * 128);

  // pass s: tile (mt, nt), the expert whose weights it uses and the 128-row
  // halves taking part (bit h for half h)
  auto tile_of = [&](int s, int* mt, int* nt, int* e, int* hm) {
    if constexpr (CONTIG) {
      dense_tile(__builtin_amdgcn_readfirstlane(pass_tile[s]), mt, nt);
      *e = __builtin_amdgcn_readfirstlane(pass_exp[s]);
      *hm = __builtin_amdgcn_readfirstlane(pass_half[s]);
    } else if constexpr (KG) {
      // round s of one tile per workgroup, XCD-contiguous inside the round
      const int t = round_tile(b, s, G, T);
      const int g = t / tpg;
      grouped_mn(t - g * tpg, p.m_tiles, p.n_tiles, GM, mt, nt);
      *e = g;  // the group (of C and D; A and B are shared)
      *hm = 3;
    } else {
      dense_tile(s, mt, nt);
      *e = 0;
      *hm = 3;
    }
  };
  // K blocks [lo, hi) of pass s (K-grouped: its group's; a group without
  // blocks runs one iteration over zero operands, zero = 1)
  auto k_range = [&](int e, int* lo, int* hi, int* zero) {
    *lo = 0;
    *hi = KB;
    *zero = 0;
    if constexpr (KG) {
      *lo = __builtin_amdgcn_readfirstlane(kpref[e]);
      *hi = __builtin_amdgcn_readfirstlane(kpref[e + 1]);
      if (*hi == *lo) {
        *zero = 1;
        *hi = *lo + 1;
      }
    }
  };

  if constexpr (KG) {
    J = 0;
    for (int s = 0; s < nseg; ++s) {
      int mt, nt, e, hm, lo, hi, z;
      tile_of(s, &mt, &nt, &e, &hm);
      k_range(e, &lo, &hi, &z);
      J += hi - lo;
    }
  }

#define WD_SLOT(st) ((st) == 0 ? slot0 : slot1)
#define WD_SS(st) (reinterpret_cast<float*>(WD_SLOT(st) + SLOT_S))

  // ---- issue pointer: iteration j + 1 of this workgroup's sequence
  int is_seg = 0, is_kb = 0, is_hi = KB, is_zero = 0;
  uint32_t is_aoff[A_INS], is_boff[B_INS], is_soff;
  const uint8_t* is_bptr = p.B;  // weights of the pass's expert
  const bool bwave = KG && wave >= 4;  // K-grouped: waves 4..7 load beta of the tile's columns
  auto is_setup = [&]() {
    int mt, nt, e, hm;
    tile_of(is_seg, &mt, &nt, &e, &hm);
    k_range(e, &is_kb, &is_hi, &is_zero);
    if (KG) e = 0;  // B is shared by the groups
    is_bptr = p.B + (size_t)e * (size_t)N * (size_t)K;
    const int row_limit = rows - mt * BM < BM ? rows - mt * BM : BM;
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int r = 64 * i + a_loc;
      bool ld = r < row_limit && ((hm >> (r >> 7)) & 1);
      // contiguous: only the rows tagged with the pass's expert (padding rows
      // and another expert's rows are never stored, so their A is not read)
      if constexpr (CONTIG) ld = ld && ((pass_mask[is_seg][r >> 5] >> (r & 31)) & 1u);
      is_aoff[i] = ld ? (uint32_t)(mt * BM + r) * (uint32_t)K + dma_chunk : kWideOOB;
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      const int c = nt * BN + 64 * i + b_perm;
      is_boff[i] = c < N ? (uint32_t)c * (uint32_t)K + dma_chunk : kWideOOB;
    }
    const int srow = wave * 64 + lane;  // alpha of the tile's rows that exist
    is_soff = srow < BM && srow < row_limit && ((hm >> (srow >> 7)) & 1) ? (uint32_t)((mt * BM + srow) * 4) : kWideOOB;
    if (bwave) {
      const int scol = nt * BN + (wave - 4) * 64 + lane;
      is_soff = scol < N ? (uint32_t)(scol * 4) : kWideOOB;
    }
  };
  is_setup();

#define WD_ISSUE_BEGIN()                                                                                   \
  const bool in_ = is_seg < nseg;                                                                          \
  const bool ld_ = in_ && !(KG && is_zero);                                                                \
  const __amdgpu_buffer_rsrc_t ra_ = wide_rsrc(p.A, ld_ ? a_bytes : 0u);                                   \
  const __amdgpu_buffer_rsrc_t rb_ = wide_rsrc(is_bptr, ld_ ? b_bytes : 0u);                               \
  const __amdgpu_buffer_rsrc_t rs_ = bwave ? wide_rsrc(p.sfb, ld_ ? (uint32_t)N * (uint32_t)KB * 4u : 0u)  \
                                           : wide_rsrc(p.sfa, ld_ ? s_bytes : 0u);                         \
  const int ks_ = is_kb << 7
#define WD_ISSUE_LOAD(st_, n_)                                                                             \
  do {                                                                                                     \
    if ((n_) < A_INS)                                                                                      \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_, (DG_LDS void*)(WD_SLOT(st_) + ((n_) * NWAVES + wave) * 1024), \
                                               16, is_aoff[(n_) < A_INS ? (n_) : 0], ks_, 0, 0);           \
    else if ((n_) < A_INS + B_INS)                                                                         \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                            \
          rb_, (DG_LDS void*)(WD_SLOT(st_) + BM * 128 + ((n_) - A_INS) * NWAVES * 1024 + wave * 1024), 16,  \
          is_boff[(n_) < A_INS + B_INS && (n_) >= A_INS ? (n_) - A_INS : 0], ks_, 0, 0);                   \
    else                                                                                                   \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_, (DG_LDS void*)(WD_SS(st_) + wave * 64), 4, is_soff,    \
                                               (UE ? (is_kb >> 2) : is_kb) * (bwave ? N : p.sfa_ld) * 4, 0, 0); \
  } while (0)
#define WD_ISSUE_END()                                                                                     \
  do {                                                                                                     \
    if (in_ && ++is_kb == is_hi) {                                                                         \
      if (++is_seg < nseg) is_setup();                                                                     \
    }                                                                                                      \
  } while (0)

  // ---- compute pointer: iteration j
  int cp_seg = 0, cp_kb = 0, cp_hi = KB, cp_zero = 0;
  int cp_mt, cp_nt, cp_e, cp_hm;
  tile_of(0, &cp_mt, &cp_nt, &cp_e, &cp_hm);
  k_range(cp_e, &cp_kb, &cp_hi, &cp_zero);
  (void)cp_zero;
  const DG_CONST float* sfb_w;
  bool cp_act;  // this wave's rows take part in the pass
  auto cp_setup = [&]() {
    cp_act = !CONTIG || ((cp_hm >> (wm >> 1)) & 1);
    int nblk = (cp_nt * BN + wn * 128) >> 7;
    nblk = nblk < NB ? nblk : NB - 1;
    const uint64_t a = reinterpret_cast<uint64_t>(p.sfb + ((int64_t)(KG ? 0 : cp_e) * NB + nblk) * (UE ? KW : KB));
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

  // deferred bf16 store of a finished tile (after the next barrier): lane l
  // of row tile i holds row wm*64 + 16 i + l % 16 and, in 64-column half h,
  // columns wn*128 + 64 h + 16 q + [0, 16).  Outside the contiguous form the
  // tile goes out through a per-wave LDS transpose, so that eight consecutive
  // lanes store one row's 128 contiguous bytes (on 4096 x 32768 x 512 the
  // store-bound call took 11% less time than with each lane storing its own
  // 16-column run of a row, 16 rows per instruction); the contiguous form,
  // whose LDS is full, stores the runs directly.
  bool pend = false;
  int st_row0 = 0, st_col0 = 0, st_grp = 0;
  uint32_t st_m[8] = {~0u, ~0u, ~0u, ~0u, ~0u, ~0u, ~0u, ~0u};  // contiguous: rows tagged with the pass's expert
#define WD_OUT_OFF(i_, h_) /* fp32 byte offset of the lane's run (row tile i_, column half h_), or OOB */ \
  ((st_row0 + wm * 64 + (i_) * 16 + q16 < rows && st_col0 + wn * 128 + (h_) * 64 + q * 16 < N)             \
       ? ((uint32_t)(st_row0 + wm * 64 + (i_) * 16 + q16) * (uint32_t)N +                                   \
          (uint32_t)(st_col0 + wn * 128 + (h_) * 64 + q * 16)) * 4u                                        \
       : kWideOOB)
#define WD_LOAD_C(cv_, i_)                                                                                 \
  _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_) {                                                       \
    const uint32_t o_ = WD_OUT_OFF(i_, h_);                                                                \
    _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_)                                                       \
      cv_[4 * h_ + j_] = HASC ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(           \
                                    rcg_, o_ == kWideOOB ? kWideOOB : o_ + 16u * j_, 0, 0))                \
                              : f32x4{0.f, 0.f, 0.f, 0.f};                                                 \
  }
#define WD_STORE_U()                                                                                       \
  do {                                                                                                     \
    if constexpr (ACC) {                                                                                   \
      /* K-grouped: C and D of the tile's group */                                                         \
      const size_t gof_ = KG ? (size_t)st_grp * (size_t)rows * (size_t)N : 0;                              \
      const __amdgpu_buffer_rsrc_t rdg_ = KG ? wide_rsrc(p.Dacc + gof_, (uint32_t)rows * (uint32_t)N * 4u) : rd; \
      const __amdgpu_buffer_rsrc_t rcg_ =                                                                  \
          KG ? wide_rsrc(HASC ? p.Cacc + gof_ : p.Cacc, HASC ? (uint32_t)rows * (uint32_t)N * 4u : 0u) : rc; \
      f32x4 ca_[TN], cb_[TN];                                                                              \
      WD_LOAD_C(ca_, 0);                                                                                   \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) {                                                  \
        f32x4* cur_ = (i_ & 1) ? cb_ : ca_;                                                                \
        f32x4* nxt_ = (i_ & 1) ? ca_ : cb_;                                                                \
        if (i_ + 1 < TM) { WD_LOAD_C(nxt_, i_ + 1); }                                                      \
        _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_) {                                                 \
          const uint32_t o_ = WD_OUT_OFF(i_, h_);                                                          \
          _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_)                                                 \
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(wu32x4, u[i_][4 * h_ + j_] + cur_[4 * h_ + j_]), \
                                                   rdg_, o_ == kWideOOB ? kWideOOB : o_ + 16u * j_, 0, 0); \
        }                                                                                                  \
      }                                                                                                    \
    } else if constexpr (!CONTIG) {                                                                        \
      /* through this wave's 2 KB of LDS, one 16-row x 64-column block at a time: lane (q, r) writes its     \
         32 bytes of row r, then lane l reads 16 bytes of row l / 8 (and 8 + l / 8) at chunk l % 8, so      \
         each store has eight consecutive lanes per 128-byte row segment (16-byte chunk c of row r at      \
         position c ^ (r % 8)) */                                                                          \
      uint8_t* stg_ = stage + wave * 2048;                                                                 \
      const int sr_ = lane >> 3;                                                                           \
      const int sc_ = lane & 7;                                                                            \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) {                                                  \
        const int ra_ = st_row0 + wm * 64 + i_ * 16 + sr_;                                                 \
        _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_) {                                                 \
          uint32_t w_[8];                                                                                  \
          _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_) {                                               \
            w_[2 * j_] = pack_bf16x2(u[i_][4 * h_ + j_][0], u[i_][4 * h_ + j_][1]);                        \
            w_[2 * j_ + 1] = pack_bf16x2(u[i_][4 * h_ + j_][2], u[i_][4 * h_ + j_][3]);                    \
          }                                                                                                \
          *reinterpret_cast<uint4*>(stg_ + q16 * 128 + (((2 * q) ^ (q16 & 7)) << 4)) =                     \
              uint4{w_[0], w_[1], w_[2], w_[3]};                                                           \
          *reinterpret_cast<uint4*>(stg_ + q16 * 128 + (((2 * q + 1) ^ (q16 & 7)) << 4)) =                 \
              uint4{w_[4], w_[5], w_[6], w_[7]};                                                           \
          const uint4 va_ = *reinterpret_cast<const uint4*>(stg_ + sr_ * 128 + ((sc_ ^ sr_) << 4));        \
          const uint4 vb_ = *reinterpret_cast<const uint4*>(stg_ + (8 + sr_) * 128 + ((sc_ ^ sr_) << 4));  \
          const int c_ = st_col0 + wn * 128 + h_ * 64 + sc_ * 8;                                           \
          const uint32_t offa_ = (ra_ < rows && c_ < N) ? ((uint32_t)ra_ * (uint32_t)N + (uint32_t)c_) * 2u : kWideOOB; \
          const uint32_t offb_ = (ra_ + 8 < rows && c_ < N) ? ((uint32_t)(ra_ + 8) * (uint32_t)N + (uint32_t)c_) * 2u : kWideOOB; \
          __builtin_amdgcn_raw_buffer_store_b128(wu32x4{va_.x, va_.y, va_.z, va_.w}, rd, offa_, 0, 0);   \
          __builtin_amdgcn_raw_buffer_store_b128(wu32x4{vb_.x, vb_.y, vb_.z, vb_.w}, rd, offb_, 0, 0);   \
        }                                                                                                  \
      }                                                                                                    \
    } else                                                                                                 \
    _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) {                                                    \
      const int rr_ = wm * 64 + i_ * 16 + q16;                                                             \
      const int r_ = st_row0 + rr_;                                                                        \
      const bool tag_ = !CONTIG || ((st_m[rr_ >> 5] >> (rr_ & 31)) & 1u);                                  \
      _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_) {                                                   \
        const int c_ = st_col0 + wn * 128 + h_ * 64 + q * 16;                                              \
        const uint32_t off_ = (r_ < rows && c_ < N && tag_) ? ((uint32_t)r_ * (uint32_t)N + (uint32_t)c_) * 2u : kWideOOB; \
        uint32_t w_[8];                                                                                    \
        _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_) {                                                 \
          w_[2 * j_] = pack_bf16x2(u[i_][4 * h_ + j_][0], u[i_][4 * h_ + j_][1]);                          \
          w_[2 * j_ + 1] = pack_bf16x2(u[i_][4 * h_ + j_][2], u[i_][4 * h_ + j_][3]);                      \
        }                                                                                                  \
        __builtin_amdgcn_raw_buffer_store_b128(wu32x4{w_[0], w_[1], w_[2], w_[3]}, rd, off_, 0, 0);        \
        __builtin_amdgcn_raw_buffer_store_b128(wu32x4{w_[4], w_[5], w_[6], w_[7]}, rd,                     \
                                               off_ == kWideOOB ? kWideOOB : off_ + 16u, 0, 0);            \
      }                                                                                                    \
    }                                                                                                      \
  } while (0)

#define WD_FRAG(dst_, base_, off_)                                                                         \
  do {                                                                                                     \
    const uint4 lo_ = *reinterpret_cast<const uint4*>((base_) + fr_lo + (off_));                          \
    const uint4 hi_ = *reinterpret_cast<const uint4*>((base_) + fr_hi + (off_));                          \
    dst_ = i32x8{(int)lo_.x, (int)lo_.y, (int)lo_.z, (int)lo_.w, (int)hi_.x, (int)hi_.y, (int)hi_.z, (int)hi_.w}; \
  } while (0)

  // One iteration jj_ in slot st_ (= jj_ % 2).  After the wait for this
  // wave's loads of jj_ and the barrier (everyone's loads of jj_ landed,
  // everyone done reading slot st_ ^ 1), a finished tile is stored, the A
  // fragments, row scales and first B fragment of jj_ are read, and the 32
  // MFMAs run j-major with the next B fragment read one fragment ahead, the
  // block's loads for jj_ + 1 (into slot st_ ^ 1) in the first steps and the
  // promotions three MFMAs behind.
#define WD_STEP(st_, jj_)                                                                                  \
  do {                                                                                                     \
    const bool live_ = (jj_) < J;                                                                          \
    const float beta_ = UE || BF16 || KG ? 1.f : (live_ ? sfb_w[cp_kb] : 0.f);                             \
    /* UE8M0: the iteration's codes sit in byte cp_kb % 4 of their packed words */                        \
    const int ash_ = 8 * (cp_kb & 3);                                                                      \
    const int bcode_ = UE && live_ ? __builtin_bit_cast(int, sfb_w[cp_kb >> 2]) >> ash_ : 0;              \
    (void)beta_;                                                                                           \
    (void)ash_;                                                                                            \
    (void)bcode_;                                                                                          \
    wait_vmcnt<0>();                                                                                       \
    wait_lgkmcnt0();                                                                                       \
    __builtin_amdgcn_s_barrier();                                                                          \
    if (pend) {                                                                                            \
      WD_STORE_U();                                                                                        \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_)                                                    \
        _Pragma("unroll") for (int j_ = 0; j_ < TN; ++j_) u[i_][j_] = f32x4{0.f, 0.f, 0.f, 0.f};           \
      pend = false;                                                                                        \
    }                                                                                                      \
    const uint8_t* sl_ = WD_SLOT(st_);                                                                     \
    if (!cp_act) { /* no rows of this wave in the pass: only this wave's share of the loads */             \
      WD_ISSUE_BEGIN();                                                                                    \
      _Pragma("unroll") for (int n_ = 0; n_ < L_BLOCK; ++n_) WD_ISSUE_LOAD((st_) ^ 1, n_);                \
      WD_ISSUE_END();                                                                                      \
    } else if constexpr (BF16) {                                                                           \
      i32x8 af_[TM];                                                                                       \
      uint4 bh_[2]; /* B half fragments, streamed one ahead */                                             \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) WD_FRAG(af_[i_], sl_ + a_row0, i_ * 2048);         \
      bh_[0] = *reinterpret_cast<const uint4*>(sl_ + b_row0 + fr_lo);                                      \
      WD_ISSUE_BEGIN();                                                                                    \
      _Pragma("unroll") for (int k_ = 0; k_ < 2 * TM * TN; ++k_) {                                         \
        const int h_ = k_ / (TM * TN);    /* 0: first 32 K elements, 1: second */                          \
        const int f_ = k_ % (TM * TN);                                                                     \
        const int j_ = f_ / TM;                                                                            \
        const int i_ = f_ % TM;                                                                            \
        const int sq_ = h_ * TN + j_;     /* position in the half-fragment stream */                       \
        if (i_ == 0 && sq_ + 1 < 2 * TN) {                                                                 \
          const int hn_ = (sq_ + 1) / TN, jn_ = (sq_ + 1) % TN;                                            \
          bh_[(sq_ + 1) & 1] = *reinterpret_cast<const uint4*>(sl_ + b_row0 + jn_ * 2048 + (hn_ ? fr_hi : fr_lo)); \
        }                                                                                                  \
        const wi32x4 av_ = h_ == 0 ? wi32x4{af_[i_][0], af_[i_][1], af_[i_][2], af_[i_][3]}                \
                                   : wi32x4{af_[i_][4], af_[i_][5], af_[i_][6], af_[i_][7]};               \
        u[i_][j_] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(wbf16x8, bh_[sq_ & 1]),     \
                                                           __builtin_bit_cast(wbf16x8, av_), u[i_][j_], 0, 0, 0); \
        if (k_ < L_BLOCK) WD_ISSUE_LOAD((st_) ^ 1, k_);                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                                 \
      }                                                                                                    \
      WD_ISSUE_END();                                                                                      \
    } else {                                                                                               \
      i32x8 af_[TM], bf_[2];                                                                               \
      float sc_[TM];  /* alpha * beta of the row tile's rows */                                            \
      int acode_[TM]; /* UE8M0: the rows' alpha codes in byte 0 */                                         \
      _Pragma("unroll") for (int i_ = 0; i_ < TM; ++i_) {                                                  \
        WD_FRAG(af_[i_], sl_ + a_row0, i_ * 2048);                                                         \
        const float al_ = WD_SS(st_)[wm * 64 + i_ * 16 + q16];                                             \
        if constexpr (UE) acode_[i_] = __builtin_bit_cast(int, al_) >> ash_;                               \
        else sc_[i_] = al_ * beta_;                                                                        \
      }                                                                                                    \
      WD_FRAG(bf_[0], sl_ + b_row0, 0);                                                                    \
      WD_ISSUE_BEGIN();                                                                                    \
      f32x4 t_[4];                                                                                         \
      f32x4 bt_[2]; /* K-grouped: beta of fragment j's columns, two j in flight */                         \
      (void)bt_;                                                                                           \
      _Pragma("unroll") for (int k_ = 0; k_ < TM * TN + 3; ++k_) {                                         \
        if (k_ < TM * TN) {                                                                                \
          const int j_ = k_ / TM;                                                                          \
          if (k_ % TM == 0 && j_ + 1 < TN) WD_FRAG(bf_[(j_ + 1) & 1], sl_ + b_row0, (j_ + 1) * 2048);      \
          if (KG && k_ % TM == 0) /* beta of the 4 columns of fragment j_ this lane holds */               \
            bt_[j_ & 1] = *reinterpret_cast<const f32x4*>(                                                 \
                WD_SS(st_) + 256 + wn * 128 + (j_ >> 2) * 64 + q * 16 + (j_ & 3) * 4);                     \
          if constexpr (UE) /* alpha and beta applied, and the scaled block product added to the */        \
            /* accumulator, by the matrix cores (exact powers of two): the promotion in one instruction */  \
            u[k_ % TM][j_] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf_[j_ & 1], af_[k_ % TM],   \
                                                                             u[k_ % TM][j_], 0, 0, 0,      \
                                                                             bcode_, 0, acode_[k_ % TM]);  \
          else                                                                                             \
            t_[k_ & 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf_[j_ & 1], af_[k_ % TM],        \
                                                                         f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0); \
          if (k_ < L_BLOCK) WD_ISSUE_LOAD((st_) ^ 1, k_);                                                  \
        }                                                                                                  \
        if (k_ >= 3) {                                                                                     \
          const int kk_ = k_ - 3;                                                                          \
          f32x4& uk_ = u[kk_ % TM][kk_ / TM];                                                              \
          if constexpr (!UE) {                                                                             \
            if constexpr (KG) t_[kk_ & 3] *= bt_[(kk_ / TM) & 1];                                          \
            _Pragma("unroll") for (int v_ = 0; v_ < 4; ++v_)                                               \
              uk_[v_] = __builtin_fmaf(t_[kk_ & 3][v_], sc_[kk_ % TM], uk_[v_]);                           \
          }                                                                                                \
          /* (UE8M0: pins the accumulator of the MFMA three steps back, which keeps the schedule) */       \
          asm volatile("" : "+v"(uk_));                                                                    \
        }                                                                                                  \
        __builtin_amdgcn_sched_barrier(0);                                                                 \
      }                                                                                                    \
      WD_ISSUE_END();                                                                                      \
    }                                                                                                      \
    if (live_ && ++cp_kb == cp_hi) { /* a tile is done */                                                 \
      st_row0 = cp_mt * BM;                                                                                \
      st_col0 = cp_nt * BN;                                                                                \
      st_grp = cp_e;                                                                                       \
      if (CONTIG) {                                                                                        \
        _Pragma("unroll") for (int w_ = 0; w_ < 8; ++w_) st_m[w_] = __builtin_amdgcn_readfirstlane(pass_mask[cp_seg][w_]); \
      }                                                                                                    \
      pend = true;                                                                                         \
      if (++cp_seg < nseg) {                                                                               \
        tile_of(cp_seg, &cp_mt, &cp_nt, &cp_e, &cp_hm);                                                    \
        k_range(cp_e, &cp_kb, &cp_hi, &cp_zero);                                                           \
        cp_setup();                                                                                        \
      }                                                                                                    \
    }                                                                                                      \
  } while (0)

  // prologue: iteration 0 into slot 0
  {
    WD_ISSUE_BEGIN();
#pragma unroll
    for (int n_ = 0; n_ < L_BLOCK; ++n_) WD_ISSUE_LOAD(0, n_);
    WD_ISSUE_END();
  }
  for (int j = 0; j < J; j += 2) {
    WD_STEP(0, j);
    WD_STEP(1, j + 1);
  }
  if (pend) WD_STORE_U();
  wait_vmcnt<0>();  // no LDS writes or stores in flight past this point
  wait_lgkmcnt0();

#undef WD_STEP
#undef WD_FRAG
#undef WD_STORE_U
#undef WD_LOAD_C
#undef WD_OUT_OFF
#undef WD_ISSUE_BEGIN
#undef WD_ISSUE_LOAD
#undef WD_ISSUE_END
#undef WD_SS
#undef WD_SLOT
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace

hipError_t launch_gemm_wide(int mode, int grid, const GemmParams& p, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (mode == kContiguous)
    hipLaunchKernelGGL((fp8_gemm_wide_kernel<kContiguous, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  else if (mode == kContiguousUe8m0)
    hipLaunchKernelGGL((fp8_gemm_wide_kernel<kContiguousUe8m0, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  else if (mode == kDenseUe8m0)
    hipLaunchKernelGGL((fp8_gemm_wide_kernel<kDenseUe8m0, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  else if (mode == kDenseBf16)
    hipLaunchKernelGGL((fp8_gemm_wide_kernel<kDenseBf16, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  else if (mode == kKGrouped && p.Cacc)
    hipLaunchKernelGGL((fp8_gemm_wide_kernel<kKGrouped, true>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  else if (mode == kKGrouped)
    hipLaunchKernelGGL((fp8_gemm_wide_kernel<kKGrouped, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  else if (mode == kDenseAcc && p.Cacc)
    hipLaunchKernelGGL((fp8_gemm_wide_kernel<kDenseAcc, true>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  else if (mode == kDenseAcc)
    hipLaunchKernelGGL((fp8_gemm_wide_kernel<kDenseAcc, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((fp8_gemm_wide_kernel<kDense, false>), dim3((unsigned)grid), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dg
